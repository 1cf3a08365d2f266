"""Automatic DP / stream-K / split-K choice and the split-K comparator (CPU).

Oracle pins, each from what the pages or the definition of split-K fix:

* the review of the "auto" default (rocm-libraries PR #13151): at the
  1216-CTA workspace pool a one-tile problem with 1024-1215 MAC iterations
  gives a stream-K partition with no stream-K CTAs, so "auto" must not pick
  stream-K there; more generally "auto" picks stream-K only when the
  partition it launches has stream-K CTAs;
* "auto" for the reduction is the workspace fix-up;
* many tiles (two or more full waves, or whole waves) or a short reduction
  keep split-K;
* split-K cuts every tile into equal K slices: checked by brute force over
  the partition's ranges (each CTA runs exactly one slice of one tile when
  the slice count divides the iterations per tile), and every MAC iteration
  is still covered once.

Then the C++ planner's resolution equals the oracle's over a sweep.
"""

import json
import os

import pytest

import implicit_gemm_conv_dp_amd as skg
from implicit_gemm_conv_dp_amd import _lib
from oracle import partition as P

TILES = {name: tuple(map(int, name.split("x"))) for name in skg.TILES}


@pytest.fixture(scope="module")
def printed(golden_dir):
    with open(os.path.join(golden_dir, "printed_values.json")) as f:
        return json.load(f)


def resolved_plan(T, ipt, mode, red, ctas, **kw):
    rm, rr, rc, S = P.resolve_launch(T, ipt, mode, red, ctas, **kw)
    return (rm, rr, rc, S), P.plan(1, T, ipt, 128, 128, 4, rm, rr, rc, **kw)


def test_auto_avoids_the_printed_all_dp_case(printed):
    d = printed["one_tile_all_dp"]
    pool = d["pool"]
    for ipt in range(d["iters_first"], d["iters_last"] + 1):
        # the page's failure: the stream-K partition itself has no SK CTAs
        assert P.plan(1, 1, ipt, 128, 128, 4, "dp_sk", "workspace", pool).sk_ctas == d["sk_ctas"]
        (rm, rr, rc, S), p = resolved_plan(1, ipt, "auto", "auto", pool)
        assert S > 1, ipt           # split-K, not the all-DP stream-K launch
        assert p.sk_ctas == S and p.dp_tiles == 0
        assert rr == "workspace"


def test_auto_stream_k_only_with_stream_k_ctas():
    for pool in (1, 7, 64, 256, 1216):
        for T in list(range(1, 40)) + [pool - 1, pool, pool + 1, 2 * pool - 1, 2 * pool, 3 * pool + 5]:
            if T < 1:
                continue
            for ipt in (1, 7, 8, 9, 64, 1100, 1568):
                (rm, rr, rc, S), p = resolved_plan(T, ipt, "auto", "auto", pool)
                assert rr == "workspace"
                if S == 1 and rm == "dp_sk":
                    # stream-K: only for a ragged wave over a long reduction,
                    # and the launched partition has stream-K CTAs
                    assert p.sk_ctas > 0 and rc == pool
                    assert T % pool != 0 and T < 2 * pool and ipt >= P.LONG_REDUCTION
                else:
                    assert rc == T * S
                if T >= 2 * pool or T % pool == 0 or ipt < P.LONG_REDUCTION:
                    assert rm == "dp" or S > 1, (pool, T, ipt)


def slices_by_brute_force(T, ipt, S):
    """Each CTA's iterations, expanded one by one from the partition."""
    rm, rr, rc, s = P.resolve_launch(T, ipt, "splitk", "workspace", S)
    p = P.plan(1, T, ipt, 128, 128, 4, rm, rr, rc)
    runs = []
    for b in range(p.sk_ctas):
        lo, hi = p.sk_range(b)
        runs.append([(it // ipt, it % ipt) for it in range(lo, hi)])
    return p, s, runs


def test_split_k_gives_equal_slices():
    for T in (1, 2, 3, 5, 12):
        for ipt in (1, 2, 8, 12, 30, 64):
            for S in range(1, ipt + 1):
                p, s, runs = slices_by_brute_force(T, ipt, S)
                assert s == S
                if S == 1:
                    assert p.mode == "dp" and p.sk_ctas == 0 and p.dp_tiles == T
                    continue
                assert p.dp_tiles == 0 and p.sk_ctas == T * S
                seen = sorted(x for r in runs for x in r)
                assert seen == [(t, k) for t in range(T) for k in range(ipt)]
                lens = [len(r) for r in runs]
                assert max(lens) - min(lens) <= 1
                if ipt % S == 0:
                    w = ipt // S
                    for b, r in enumerate(runs):
                        t, j = divmod(b, S)
                        assert r == [(t, k) for k in range(j * w, (j + 1) * w)], (T, ipt, S, b)


def test_split_k_explicit_slices_clamp_and_default():
    assert P.resolve_launch(4, 6, "splitk", "tree", 50) == ("dp_sk", "tree", 24, 6)
    assert P.resolve_launch(4, 6, "splitk", "tree", 1) == ("dp", "tree", 4, 1)
    # default: fill the pool, slices of at least LONG_REDUCTION iterations
    assert P.resolve_launch(1, 1100, "splitk", "workspace", -1, num_cus=304,
                            resident_per_cu=8) == ("dp_sk", "workspace", 137, 137)
    assert P.resolve_launch(36, 1568, "splitk", "workspace", -1, num_cus=256,
                            resident_per_cu=2) == ("dp_sk", "workspace", 36 * 14, 14)
    assert P.resolve_launch(304, 64, "splitk", "tree", -1, num_cus=256,
                            resident_per_cu=1) == ("dp", "tree", 304, 1)


def test_workloads_auto_choice():
    # few filter tiles over a very long reduction (a wgrad): stream-K
    assert P.resolve_launch(36, 1568, "auto", "auto", -1, num_cus=256,
                            resident_per_cu=2)[0:2] == ("dp_sk", "workspace")
    # 19 x 16 tiles at 256 CUs: a ragged second wave over 64 iterations
    assert P.resolve_launch(304, 64, "auto", "auto", -1, num_cus=256,
                            resident_per_cu=1) == ("dp_sk", "workspace", 256, 1)
    # 32 x 32 tiles fill whole waves of 256: no stream-K, no split
    assert P.resolve_launch(1024, 64, "auto", "auto", -1, num_cus=256,
                            resident_per_cu=1) == ("dp", "workspace", 1024, 1)


def test_forced_modes_pass_through():
    for m in P.MODES:
        for r in P.REDUCTIONS:
            assert P.resolve_launch(10, 20, m, r, 7) == (m, r, 7, 1)
    assert P.resolve_launch(10, 20, "dp_sk", "auto", 7) == ("dp_sk", "workspace", 7, 1)
    with pytest.raises(ValueError):
        P.resolve_launch(10, 20, "bogus", "tree", 7)
    with pytest.raises(ValueError):
        P.resolve_launch(10, 20, "auto", "bogus", 7)
    with pytest.raises(ValueError):
        P.resolve_launch(10, 20, "splitk", "tree", 0)


FIELDS = ["tiles_m", "tiles_n", "tiles", "iters_per_tile", "pool", "dp_tiles", "sk_tiles",
          "sk_ctas", "sk_iters", "iters_per_sk_cta", "extra_iters", "grid", "max_contrib",
          "linear_partners", "tree_rounds", "flags_bytes", "partials_bytes", "workspace_bytes"]


def check_same(c, tiles, tm, tn, mode, red, ctas):
    T = tiles[0] * tiles[1]
    rm, rr, rc, S = P.resolve_launch(T, tiles[2], mode, red, ctas)
    o = P.plan(*tiles, tm, tn, 4, rm, rr, rc)
    for f in FIELDS:
        assert c[f] == getattr(o, f), (f, c[f], getattr(o, f), mode, red, ctas)
    assert c["mode"] == _lib.MODES[rm] and c["reduction"] == _lib.REDUCTIONS[rr]
    assert c["requested_mode"] == _lib.MODES[mode] and c["slices"] == S


@pytest.mark.parametrize("tile,dt", [("128x128x32", "f16"), ("256x256x64", "bf16"),
                                     ("256x256x128", "e4m3")])
def test_gemm_resolution_equals_oracle(tile, dt):
    tm, tn, tk = TILES[tile]
    n = 0
    for M in (1, tm, 3 * tm + 5, 4864):
        for N in (16, 2 * tn + 8, 4096):
            for K in (tk, 9 * tk, 4096 + tk):
                for mode in ("splitk", "auto"):
                    for red in ("linear", "tree", "workspace", "auto"):
                        for ctas in (1, 3, 6, 77, 256, 1216):
                            c = skg.plan_gemm(M=M, N=N, K=K, dtype_ab=dt, dtype_c="bf16",
                                              tile=tile, mode=mode, reduction=red, ctas=ctas)
                            check_same(c, P.gemm_tiles(M, N, K, tm, tn, tk), tm, tn, mode, red,
                                       ctas)
                            n += 1
    assert n > 500


def test_wgrad_resolution_equals_oracle():
    tm, tn, tk = TILES["128x128x64"]
    for (n, h, w, c, k, st, g) in [(32, 56, 56, 256, 256, (1, 1), 1), (64, 28, 28, 512, 512, (2, 2), 32),
                                   (2, 9, 9, 16, 24, (1, 1), 1)]:
        for mode in ("splitk", "auto"):
            for red in ("tree", "workspace", "auto"):
                for ctas in (2, 11, 256, 1024):
                    cp = skg.plan_wgrad(n=n, h=h, w=w, c=c, k=k, r=3, s=3, stride=st,
                                        pad=(1, 1), groups=g, dtype="bf16", tile="128x128x64",
                                        mode=mode, reduction=red, ctas=ctas)
                    tiles = P.wgrad_tiles(n, h, w, c, k, 3, 3, st[0], st[1], 1, 1, g, tm, tn, tk)
                    check_same(cp, tiles, tm, tn, mode, red, ctas)


def test_split_k_rejects_bad_slices():
    for bad in (0, -2):
        with pytest.raises(skg.SkgError) as ei:
            skg.plan_gemm(M=256, N=256, K=4096, dtype_ab="f16", dtype_c="f16",
                          tile="128x128x32", mode="splitk", reduction="workspace", ctas=bad)
        assert ei.value.status == -2
