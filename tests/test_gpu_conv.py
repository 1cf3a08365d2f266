"""GPU parity of the forward convolution and input gradient (dgrad) as
implicit GEMMs on the stream-K engine, against the oracle (through the C ABI).

Dense, strided (dgrad: taps that reach no output pixel), grouped and
rectangular shapes with partial M and N tiles and reduction tails; every
conv tile x launch mode x fix-up; random data within 5e-3 (bf16 or f16
outputs, fp32 accumulate) and integer-exact data bit for bit (fp32 outputs);
the layer shapes of the two wgrad workloads at full size in the benchmark's
launch of each op.
"""

import numpy as np
import pytest
import torch

import implicit_gemm_conv_dp_amd as skg
from implicit_gemm_conv_dp_amd import synth
from oracle.conv import dgrad as oracle_dgrad, forward as oracle_forward
from oracle.wgrad import out_size

from helpers import assert_close, decode_out, out_buffer, to_dev

pytestmark = pytest.mark.gpu

MODES = ["dp", "dp_sk", "persistent"]
REDS = ["linear", "tree", "atomic", "workspace"]
TILES = ["256x256x64", "128x128x64", "256x128x64"]

# N, H, W, C, K, R, S, stride, pad, groups
SHAPES = {
    "dense": (2, 9, 9, 16, 24, 3, 3, (1, 1), (1, 1), 1),
    "strided": (3, 11, 10, 32, 16, 3, 3, (2, 2), (1, 1), 1),
    "grouped": (2, 12, 12, 64, 32, 3, 3, (2, 2), (1, 1), 4),
    "wide": (1, 17, 15, 144, 40, 3, 2, (1, 2), (1, 0), 1),
    "deep": (2, 8, 8, 264, 136, 3, 3, (1, 1), (1, 1), 1),
    # 1x1 over 16 channels: a 32-byte forward reduction, shorter than one LDS row
    "c16_1x1": (2, 5, 7, 16, 24, 1, 1, (1, 1), (0, 0), 1),
}


def inputs(op, shape, fmt, integer, seed):
    n, h, w, c, k, r, s, st, pd, g = shape
    ho, wo = out_size(h, w, r, s, st[0], st[1], pd[0], pd[1])
    na = n * h * w * c if op == "fwd" else n * ho * wo * k
    nw = k * r * s * (c // g)
    if integer:
        act = synth.integer_codes(fmt, na, seed, 0.5)
        filt = synth.integer_codes(fmt, nw, seed + 1, 0.5)
    else:
        act = synth.to_codes(synth.draw("uniform", na, seed), fmt)
        filt = synth.to_codes(synth.draw("uniform", nw, seed + 1), fmt)
    if op == "fwd":
        R = oracle_forward(fmt, act, filt, n, h, w, c, k, r, s, st[0], st[1], pd[0], pd[1], g)
    else:
        R = oracle_dgrad(fmt, act, filt, n, h, w, c, k, r, s, st[0], st[1], pd[0], pd[1], g)
    return act, filt, R.reshape(-1, R.shape[-1])


def run(op, act, filt, shape, fmt, fmt_out, tile, mode, red, ctas, ws=None):
    n, h, w, c, k, r, s, st, pd, g = shape
    ho, wo = out_size(h, w, r, s, st[0], st[1], pd[0], pd[1])
    nout = n * ho * wo * k if op == "fwd" else n * h * w * c
    out = out_buffer(fmt_out, nout)
    call = skg.fwd if op == "fwd" else skg.dgrad
    plan = call(to_dev(act, fmt), to_dev(filt, fmt), out, workspace=ws, n=n, h=h, w=w, c=c, k=k,
                r=r, s=s, stride=st, pad=pd, groups=g, dtype=fmt, dtype_out=fmt_out, tile=tile,
                mode=mode, reduction=red, ctas=ctas)
    torch.cuda.synchronize()
    cols = k if op == "fwd" else c
    return decode_out(out, fmt_out).reshape(-1, cols), plan


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("op", ["fwd", "dgrad"])
def test_random_all_modes_and_fixups(op, name, tile):
    shape = SHAPES[name]
    fmt = "bf16" if name in ("grouped", "wide") else "f16"
    act, filt, R = inputs(op, shape, fmt, False, 5)
    k = 0
    for mode in MODES:
        for red in REDS:
            if mode == "dp" and red != "linear":
                continue
            for ctas in (3, 5, 11):
                fmt_out = "f32" if red == "atomic" else ("bf16", "f16", "f32")[k % 3]
                k += 1
                Y, plan = run(op, act, filt, shape, fmt, fmt_out, tile, mode, red, ctas)
                assert_close(Y, R, fmt, "%s %s %s %s %s ctas=%d -> %s" % (op, name, tile, mode, red,
                                                                         ctas, fmt_out))
                if mode == "dp":
                    break


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("op", ["fwd", "dgrad"])
def test_integer_exact_all_modes_and_fixups(op, name, tile):
    shape = SHAPES[name]
    act, filt, R = inputs(op, shape, "bf16", True, 31)
    assert np.array_equal(R.astype(np.float32).astype(np.float64), R)
    for mode in MODES:
        for red in REDS:
            if mode == "dp" and red != "linear":
                continue
            Y, plan = run(op, act, filt, shape, "bf16", "f32", tile, mode, red, 7)
            if mode != "dp":
                assert plan["sk_ctas"] in (0, 7)
            assert np.array_equal(Y, R), "%s %s %s %s %s not bit-exact" % (op, name, tile, mode, red)


def test_plans_reach_shared_tiles():
    # The matrix above must exercise stream-K tiles shared by several CTAs.
    n, h, w, c, k, r, s, st, pd, g = SHAPES["deep"]
    for call in (skg.plan_fwd, skg.plan_dgrad):
        p = call(n=n, h=h, w=w, c=c, k=k, r=r, s=s, stride=st, pad=pd, groups=g, dtype="bf16",
                 dtype_out="f32", tile="128x128x64", mode="dp_sk", reduction="tree", ctas=7)
        assert p["sk_ctas"] == 7 and p["max_contrib"] >= 2, p


LAYERS = {
    "n32_56x56_c256_k256_3x3": (32, 56, 56, 256, 256, 3, 3, (1, 1), (1, 1), 1, "f16"),
    "n64_28x28_c512_k512_g32_3x3_s2": (64, 28, 28, 512, 512, 3, 3, (2, 2), (1, 1), 32, "bf16"),
}


@pytest.mark.parametrize("layer", list(LAYERS))
@pytest.mark.parametrize("op", ["fwd", "dgrad"])
def test_layer_full_size(op, layer):
    *shape, fmt = LAYERS[layer]
    shape = tuple(shape)
    n, h, w, c, k, r, s, st, pd, g = shape
    ho, wo = out_size(h, w, r, s, st[0], st[1], pd[0], pd[1])
    na = n * h * w * c if op == "fwd" else n * ho * wo * k
    act = synth.to_codes(synth.draw("uniform", na, 91), fmt)
    filt = synth.to_codes(synth.draw("uniform", k * r * s * (c // g), 92), fmt)
    if op == "fwd":
        R = oracle_forward(fmt, act, filt, n, h, w, c, k, r, s, st[0], st[1], pd[0], pd[1], g)
    else:
        R = oracle_dgrad(fmt, act, filt, n, h, w, c, k, r, s, st[0], st[1], pd[0], pd[1], g)
    R = R.reshape(-1, R.shape[-1])
    tile = "256x256x64" if g == 1 else "128x128x64"
    for mode, red in (("dp_sk", "tree"), ("persistent", "workspace")):
        Y, plan = run(op, act, filt, shape, fmt, "f32", tile, mode, red, 256)
        assert_close(Y, R, fmt, "%s %s %s %s" % (op, layer, mode, red))


# Block-diagonal grouped tile (16 input and 16 output channels per group,
# four groups per 64-channel N tile, two filter taps per MAC iteration).
BD_TILE = "128x64x32"
BD_SHAPES = {
    # 2 N tiles, stride 1, 128-pixel M tiles with a ragged tail (4*10*10)
    "bd_two_tiles": (4, 10, 10, 128, 128, 3, 3, (1, 1), (1, 1), 8),
    # 4 + 2 groups (ragged last N tile)
    "bd_ragged": (3, 9, 9, 96, 96, 3, 3, (1, 1), (1, 1), 6),
    # stride 2 with padding, like the grouped layer (dgrad: taps that reach
    # no output pixel)
    "bd_strided": (4, 14, 14, 64, 64, 3, 3, (2, 2), (1, 1), 4),
    # one group, uneven padding
    "bd_one_group": (3, 7, 5, 16, 16, 3, 3, (1, 1), (0, 1), 1),
    # 1x1: one tap, the second tap of the only iteration past R*S
    "bd_1x1": (2, 8, 8, 64, 64, 1, 1, (1, 1), (0, 0), 4),
    # 5x5 over 13 iterations, strides 2 x 1
    "bd_5x5": (2, 11, 9, 80, 80, 5, 5, (2, 1), (2, 2), 5),
    # dgrad stride phases: 1x1 with stride 2 (three of four phases meet no
    # tap: zero rows), stride 3 (nine phases of one tap each), 4x4 with
    # strides 2 x 3 (phases of 2 x 2 and 2 x 1 taps)
    "bd_s2_1x1": (2, 9, 8, 64, 64, 1, 1, (2, 2), (0, 0), 4),
    "bd_s3": (2, 13, 11, 48, 48, 3, 3, (3, 3), (1, 1), 3),
    "bd_s23_4x4": (2, 10, 9, 64, 64, 4, 4, (2, 3), (1, 1), 4),
}


@pytest.mark.parametrize("name", list(BD_SHAPES))
@pytest.mark.parametrize("op", ["fwd", "dgrad"])
def test_block_diagonal_integer_exact_all_modes_and_fixups(op, name):
    shape = BD_SHAPES[name]
    act, filt, R = inputs(op, shape, "bf16", True, 151)
    for mode in MODES:
        for red in REDS:
            if mode == "dp" and red != "linear":
                continue
            for ctas in (3, 7, 16):
                Y, plan = run(op, act, filt, shape, "bf16", "f32", BD_TILE, mode, red, ctas)
                assert np.array_equal(Y, R), "%s %s %s %s ctas=%d not bit-exact" % (op, name, mode,
                                                                                    red, ctas)
                if mode == "dp":
                    break


@pytest.mark.parametrize("name", ["bd_strided", "bd_s23_4x4"])
def test_block_diagonal_dgrad_empty_segments(name):
    # Split-K in 2 slices: every tile's second contributor runs MAC iteration
    # 1, which a stride phase with taps for one iteration only does not have,
    # so many stream-K segments run no iteration and hand on zeros; every
    # fix-up stays bit-exact.
    shape = BD_SHAPES[name]
    act, filt, R = inputs("dgrad", shape, "bf16", True, 167)
    for red in ("linear", "tree", "scatter", "atomic", "workspace"):
        Y, plan = run("dgrad", act, filt, shape, "bf16", "f32", BD_TILE, "splitk", red, 2)
        assert plan["iters_per_tile"] == 2 and plan["sk_ctas"] == 2 * plan["tiles"], plan
        assert np.array_equal(Y, R), "%s %s not bit-exact" % (name, red)


@pytest.mark.parametrize("tile", [BD_TILE, "128x128x64"])
@pytest.mark.parametrize("op", ["fwd", "dgrad"])
def test_data_parallel_plan_same_bits_for_every_reduction(op, tile):
    # All-DP plans run no fix-up: every reduction name (and the kernel
    # family it selects) gives the same output, in dp mode and in
    # persistent mode with a pool that divides the tiles (on the
    # block-diagonal tile the ring then streams across a CTA's tiles).
    shape = BD_SHAPES["bd_s23_4x4"] if tile == BD_TILE else SHAPES["grouped"]
    act, filt, _ = inputs(op, shape, "bf16", False, 163)
    _, p0 = run(op, act, filt, shape, "bf16", "f32", tile, "dp", "linear", 1)
    T = p0["tiles"]
    ref = None
    for mode, ctas in [("dp", 1)] + [("persistent", d) for d in sorted({T, max(1, T // 3)}) if T % d == 0]:
        for red in REDS:
            Y, plan = run(op, act, filt, shape, "bf16", "f32", tile, mode, red, ctas)
            assert plan["sk_ctas"] == 0 and plan["dp_tiles"] == T, (mode, red, ctas, plan)
            if ref is None:
                ref = Y
            assert np.array_equal(Y, ref), "%s %s %s %s ctas=%d" % (op, tile, mode, red, ctas)


@pytest.mark.parametrize("name", list(BD_SHAPES))
@pytest.mark.parametrize("op", ["fwd", "dgrad"])
def test_block_diagonal_random_16bit_outputs(op, name):
    shape = BD_SHAPES[name]
    for fmt in ("f16", "bf16"):
        act, filt, R = inputs(op, shape, fmt, False, 157)
        for mode, red, ctas, fmt_out in [("dp", "linear", 1, fmt), ("dp_sk", "tree", 5, "bf16"),
                                         ("persistent", "linear", 11, "f16"),
                                         ("persistent", "workspace", 9, fmt),
                                         ("dp_sk", "atomic", 6, "f32")]:
            Y, plan = run(op, act, filt, shape, fmt, fmt_out, BD_TILE, mode, red, ctas)
            assert_close(Y, R, fmt, "%s %s %s %s %s -> %s" % (op, name, fmt, mode, red, fmt_out))


@pytest.mark.parametrize("op", ["fwd", "dgrad"])
def test_block_diagonal_grouped_layer_full_size(op):
    # The grouped 28x28 layer (N=64, 32 groups, stride 2) on the
    # block-diagonal tile, element by element against the oracle.
    *shape, fmt = LAYERS["n64_28x28_c512_k512_g32_3x3_s2"]
    shape = tuple(shape)
    n, h, w, c, k, r, s, st, pd, g = shape
    ho, wo = out_size(h, w, r, s, st[0], st[1], pd[0], pd[1])
    na = n * h * w * c if op == "fwd" else n * ho * wo * k
    act = synth.to_codes(synth.draw("uniform", na, 91), fmt)
    filt = synth.to_codes(synth.draw("uniform", k * r * s * (c // g), 92), fmt)
    if op == "fwd":
        R = oracle_forward(fmt, act, filt, n, h, w, c, k, r, s, st[0], st[1], pd[0], pd[1], g)
    else:
        R = oracle_dgrad(fmt, act, filt, n, h, w, c, k, r, s, st[0], st[1], pd[0], pd[1], g)
    R = R.reshape(-1, R.shape[-1])
    for mode, red, fmt_out in (("persistent", "tree", "bf16"), ("dp_sk", "linear", "f32"),
                               ("dp", "linear", "bf16")):
        Y, plan = run(op, act, filt, shape, fmt, fmt_out, BD_TILE, mode, red, 256)
        assert plan["tiles_n"] == 8
        assert_close(Y, R, fmt, "%s %s %s %s -> %s" % (op, BD_TILE, mode, red, fmt_out))
