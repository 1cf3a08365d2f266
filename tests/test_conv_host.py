"""CPU tests of the forward-convolution / dgrad host side (no GPU): plans
equal the oracle partitioner on the conv tile counts field by field (the
dgrad plan adds the transposed filter after the fix-up region), and
unsupported arguments are rejected with -2 and a reason."""

import pytest

import implicit_gemm_conv_dp_amd as skg
from oracle import partition as P

from test_host_library import FIELDS, TILES

SHAPES = [
    # N, H, W, C, K, R, S, stride, pad, groups
    (32, 56, 56, 256, 256, 3, 3, (1, 1), (1, 1), 1),
    (64, 28, 28, 512, 512, 3, 3, (2, 2), (1, 1), 32),
    (2, 9, 9, 16, 24, 3, 3, (1, 1), (1, 1), 1),
    (3, 11, 10, 32, 16, 3, 3, (2, 2), (1, 1), 1),
    (1, 17, 15, 144, 40, 3, 2, (1, 2), (1, 0), 1),
]


def kw_of(shape, tile, mode, red, ctas, dtype_out="f32"):
    n, h, w, c, k, r, s, st, pd, g = shape
    return dict(n=n, h=h, w=w, c=c, k=k, r=r, s=s, stride=st, pad=pd, groups=g, dtype="bf16",
                dtype_out=dtype_out, tile=tile, mode=mode, reduction=red, ctas=ctas)


@pytest.mark.parametrize("op", ["fwd", "dgrad"])
def test_conv_plans_equal_oracle(op):
    n_checked = 0
    for shape in SHAPES:
        n, h, w, c, k, r, s, st, pd, g = shape
        for tile in ("256x256x64", "128x128x64", "256x128x64"):
            tm, tn, tk = TILES[tile]
            tiles_of = P.fwd_tiles if op == "fwd" else P.dgrad_tiles
            t = tiles_of(n, h, w, c, k, r, s, st[0], st[1], pd[0], pd[1], g, tm, tn, tk)
            for mode in ("dp", "dp_sk", "persistent"):
                for red in ("linear", "tree", "atomic", "workspace"):
                    for ctas in (7, 256, 1024):
                        kw = kw_of(shape, tile, mode, red, ctas)
                        c_plan = (skg.plan_fwd if op == "fwd" else skg.plan_dgrad)(**kw)
                        o = P.plan(*t, tm, tn, 4, mode, red, ctas)
                        aux = 0 if op == "fwd" else -(-k * r * s * (c // g) * 2 // 256) * 256
                        assert c_plan["aux_bytes"] == aux
                        for f in FIELDS:
                            v = c_plan[f] - (aux if f == "workspace_bytes" else 0)
                            assert v == getattr(o, f), (op, shape, tile, mode, red, ctas, f)
                        n_checked += 1
    assert n_checked > 500


BD_SHAPES = [
    (64, 28, 28, 512, 512, 3, 3, (2, 2), (1, 1), 32),
    (2, 9, 9, 96, 96, 3, 3, (1, 1), (1, 1), 6),
    (3, 7, 5, 16, 16, 3, 3, (1, 1), (0, 1), 1),
    (2, 8, 8, 64, 64, 1, 1, (1, 1), (0, 0), 4),
    (2, 11, 9, 80, 80, 5, 5, (2, 1), (2, 2), 5),
]


@pytest.mark.parametrize("op", ["fwd", "dgrad"])
def test_block_diagonal_conv_plans_equal_oracle(op):
    tm, tn, tk = TILES["128x64x32"]
    tiles_of = P.fwd_tiles if op == "fwd" else P.dgrad_tiles
    for shape in BD_SHAPES:
        n, h, w, c, k, r, s, st, pd, g = shape
        t = tiles_of(n, h, w, c, k, r, s, st[0], st[1], pd[0], pd[1], g, tm, tn, tk,
                     group_block=4)
        for mode in ("dp", "dp_sk", "persistent"):
            for red in ("linear", "tree", "atomic", "workspace"):
                for ctas in (7, 256):
                    kw = kw_of(shape, "128x64x32", mode, red, ctas)
                    c_plan = (skg.plan_fwd if op == "fwd" else skg.plan_dgrad)(**kw)
                    o = P.plan(*t, tm, tn, 4, mode, red, ctas)
                    aux = 0 if op == "fwd" else -(-k * r * s * (c // g) * 2 // 256) * 256
                    for f in FIELDS:
                        v = c_plan[f] - (aux if f == "workspace_bytes" else 0)
                        assert v == getattr(o, f), (op, shape, mode, red, ctas, f)
    kw = kw_of((2, 8, 8, 64, 128, 3, 3, (1, 1), (1, 1), 4), "128x64x32", "dp_sk", "tree", 8)
    assert "16 input and 16 output channels" in rejected(op, **kw)
    # dgrad runs phase by phase: at most 16 stride phases
    kw = kw_of((1, 40, 40, 64, 64, 3, 3, (5, 4), (1, 1), 4), "128x64x32", "dp_sk", "tree", 8)
    if op == "dgrad":
        assert "phases" in rejected(op, **kw)
    else:
        (skg.plan_fwd)(**kw)


def rejected(op, **kw):
    with pytest.raises(skg.SkgError) as ei:
        (skg.plan_fwd if op == "fwd" else skg.plan_dgrad)(**kw)
    assert ei.value.status == -2
    return ei.value.msg


@pytest.mark.parametrize("op", ["fwd", "dgrad"])
def test_conv_rejections(op):
    base = kw_of(SHAPES[2], "128x128x64", "dp_sk", "linear", 7)
    assert "convolution instance" in rejected(op, **dict(base, tile="128x128x32"))
    assert "convolution instance" in rejected(op, **dict(base, tile="32x64x64"))
    assert "dtype" in rejected(op, **dict(base, dtype="e4m3"))
    assert "fp32" in rejected(op, **dict(base, reduction="atomic", dtype_out="bf16"))
    assert "multiples of 8" in rejected(op, **dict(base, c=12, groups=1))
    assert "groups" in rejected(op, **dict(base, groups=3))
    assert "empty" in rejected(op, **dict(base, h=1, pad=(0, 0)))
    assert "ctas" in rejected(op, **dict(base, ctas=0))
