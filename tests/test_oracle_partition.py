"""Pins of the oracle partitioner and dispatch simulator (CPU only).

* Values the pages print (tests/golden/printed_values.json, each cited).
* Brute force over every small problem: each MAC iteration covered exactly
  once, contiguous and balanced stream-K ranges, at most one non-owner tile per
  stream-K CTA, the contributor bound, a safe all-DP plan.
* The invariant checker itself is shown to catch planted mistakes (a plan with
  an off-by-one range, a wrong inverse map), so a passing sweep means
  something.
* The dispatch model: waits only target higher block ids, every plan completes
  when the pool is resident.
"""

import json
import os
from dataclasses import replace

import pytest

from oracle import partition as P
from oracle import simulate as S


@pytest.fixture(scope="module")
def printed(golden_dir):
    with open(os.path.join(golden_dir, "printed_values.json")) as f:
        return json.load(f)


def test_default_pool_printed(printed):
    d = printed["default_pool_workspace"]
    assert P.default_pool("workspace", d["num_cus"], 8) == d["pool"]
    assert P.default_pool("atomic", d["num_cus"], 8) == d["pool"]
    assert P.default_pool("linear", 256, 8) == 256
    assert P.default_pool("tree", 256, 1) == 256
    # capped by what stays resident
    assert P.default_pool("workspace", 256, 2) == 512


def test_one_tile_short_reduction_is_all_dp(printed):
    d = printed["one_tile_all_dp"]
    for ipt in (d["iters_first"], d["iters_last"]):
        p = P.plan(1, 1, ipt, 128, 128, 4, "dp_sk", "workspace", d["pool"])
        assert p.sk_ctas == d["sk_ctas"] and p.dp_tiles == 1 and p.grid == 1
        assert p.workspace_bytes == 0 and p.iters_per_sk_cta == 1
    p = P.plan(1, 1, d["iters_last"] + 1, 128, 128, 4, "dp_sk", "workspace", d["pool"])
    assert p.sk_ctas == d["pool"]


def test_flag_table_printed(printed):
    d = printed["flag_table_bytes"]
    # A shape with a stream-K remainder under the 256-CTA pool.
    p = P.plan(19, 16, 64, 256, 256, d["n_waves"], "dp_sk", "tree", d["pool"])
    assert p.sk_ctas == d["pool"]
    assert p.flags_bytes == d["bytes_per_wave_flags"]
    assert P.ceil_div(4 * p.sk_ctas, 256) * 256 == d["bytes_per_cta_flags"]


def test_four_contributors_two_rounds(printed):
    d = printed["tree_rounds_four_ctas"]
    # one tile of 8 iterations over 4 CTAs: every CTA takes 2 iterations
    p = P.plan(1, 1, 8, 64, 64, 4, "dp_sk", "tree", 4)
    assert p.max_contrib == d["contributors"] and p.tree_rounds == d["tree_rounds"]
    assert p.linear_partners == 3


def test_small_gemm_plan_ranges():
    # 256x256x4096 GEMM, 128x128x32 tiles, 6-CTA pool, linear.
    tm, tn, ipt = P.gemm_tiles(256, 256, 4096, 128, 128, 32)
    p = P.plan(tm, tn, ipt, 128, 128, 4, "dp_sk", "linear", 6)
    assert (p.tiles, p.iters_per_tile, p.dp_tiles, p.sk_tiles, p.sk_ctas) == (4, 128, 0, 4, 6)
    assert (p.iters_per_sk_cta, p.extra_iters, p.grid) == (85, 2, 6)
    assert [p.sk_range(b) for b in range(6)] == [
        (0, 86), (86, 172), (172, 257), (257, 342), (342, 427), (427, 512)]
    assert p.contributors(2) == [2, 3, 4]
    assert p.segments(2) == [(1, 44, 128, False, True), (2, 0, 1, True, False)]
    assert p.max_contrib == 3 and p.flags_bytes == 256
    assert p.partials_bytes == 6 * 128 * 128 * 4


def test_large_gemm_plan():
    tm, tn, ipt = P.gemm_tiles(4864, 4096, 4096, 256, 256, 64)
    p = P.plan(tm, tn, ipt, 256, 256, 4, "dp_sk", "tree", 256)
    assert (p.tiles, p.dp_tiles, p.sk_tiles, p.sk_ctas, p.iters_per_sk_cta, p.extra_iters) == \
        (304, 256, 48, 256, 12, 0)
    assert p.grid == 512 and p.max_contrib == 6 and p.tree_rounds == 3
    q = P.plan(tm, tn, ipt, 256, 256, 4, "persistent", "tree", 256)
    assert q.grid == 256


def test_wgrad_tiles_fold_groups():
    # 32 groups of 16 output channels with a 32-row tile: one partial M tile
    # per group; GEMM-N = 16*3*3 = 144 -> 3 tiles of 64; Ho = Wo = 14.
    assert P.wgrad_tiles(64, 28, 28, 512, 512, 3, 3, 2, 2, 1, 1, 32, 32, 64, 64) == (32, 3, 196)
    assert P.wgrad_tiles(32, 56, 56, 256, 256, 3, 3, 1, 1, 1, 1, 1, 128, 128, 32) == (2, 18, 3136)


def bd_tiles_by_brute_force(K, groups, cpg_rs, tm, tn, gb):
    """Tiles of a block-diagonal wgrad found by walking every dW element:
    output channel k belongs to group k // Kpg, and the tile holding it is
    the one holding its group among consecutive runs of gb groups."""
    kpg = K // groups
    tiles = set()
    for k in range(K):
        for n in range(cpg_rs):
            tiles.add(((k // kpg) // gb, n // tn))
    rows = {}
    for (i, _) in tiles:
        rows[i] = [k for k in range(K) if (k // kpg) // gb == i]
    for i, ks in rows.items():
        # a tile's rows are whole groups, at most tm of them, contiguous
        assert len(ks) <= tm and ks == list(range(ks[0], ks[0] + len(ks)))
        assert len(ks) % kpg == 0
    tm_count = len({i for (i, _) in tiles})
    tn_count = len({j for (_, j) in tiles})
    assert len(tiles) == tm_count * tn_count
    return tm_count, tn_count


def test_wgrad_tiles_block_diagonal():
    # 32 groups of 16: four groups per 64-row tile -> 8 M tiles; the 144
    # columns (3x3 taps of 16 channels) in one 144-wide N tile; reduction
    # 64*14*14 in steps of 32.
    assert P.wgrad_tiles(64, 28, 28, 512, 512, 3, 3, 2, 2, 1, 1, 32, 64, 144, 32,
                         group_block=4) == (8, 1, 392)
    for groups in (1, 3, 4, 5, 6, 9, 32):
        for r, s in ((1, 1), (3, 3), (5, 5)):
            K = C = 16 * groups
            t = P.wgrad_tiles(2, 9, 9, C, K, r, s, 1, 1, r // 2, s // 2, groups, 64, 144, 32,
                              group_block=4)
            assert t[:2] == bd_tiles_by_brute_force(K, groups, 16 * r * s, 64, 144, 4)
    # one group per tile and tm = Kpg is the per-group count
    assert P.wgrad_tiles(4, 8, 8, 64, 64, 3, 3, 1, 1, 1, 1, 4, 16, 144, 32, group_block=1) == \
        P.wgrad_tiles(4, 8, 8, 64, 64, 3, 3, 1, 1, 1, 1, 4, 16, 144, 32)
    with pytest.raises(ValueError):
        P.wgrad_tiles(4, 8, 8, 64, 64, 3, 3, 1, 1, 1, 1, 4, 32, 144, 32, group_block=4)


def test_conv_tiles_block_diagonal():
    # Forward / dgrad: GEMM-N runs over channels; a block-diagonal tile of
    # 64 columns holds four whole 16-channel groups.  Brute force over every
    # output channel, as for the wgrad rows.
    for groups in (1, 3, 4, 5, 32):
        C = K = 16 * groups
        seen = {(ch // 16) // 4 for ch in range(K)}
        t = P.fwd_tiles(2, 9, 9, C, K, 3, 3, 2, 2, 1, 1, groups, 128, 64, 32, group_block=4)
        assert t[1] == len(seen)
        assert t[2] == 5  # 3*3*16 = 144 reduction elements per group, 32 per iteration
        t = P.dgrad_tiles(2, 9, 9, C, K, 3, 3, 2, 2, 1, 1, groups, 128, 64, 32, group_block=4)
        assert t[1] == len(seen) and t[2] == 2  # at most 2 x 2 taps of one stride phase
    # the workload's layers: 64 x 14 x 14 output pixels (forward), 64 x 28 x 28
    # input pixels (dgrad), 32 groups
    assert P.fwd_tiles(64, 28, 28, 512, 512, 3, 3, 2, 2, 1, 1, 32, 128, 64, 32,
                       group_block=4) == (98, 8, 5)
    # dgrad: four stride phases of 14 x 14 pixels per image (12544 pixels
    # each over 64 images, 98 tiles of 128), at most 2 x 2 taps -> 64
    # reduction elements per group
    assert P.dgrad_tiles(64, 28, 28, 512, 512, 3, 3, 2, 2, 1, 1, 32, 128, 64, 32,
                         group_block=4) == (4 * 98, 8, 2)
    with pytest.raises(ValueError):
        P.fwd_tiles(2, 9, 9, 64, 64, 3, 3, 1, 1, 1, 1, 4, 128, 128, 32, group_block=4)


def test_all_dp_plan_has_safe_divisor():
    p = P.plan(4, 4, 10, 64, 64, 4, "dp_sk", "linear", 16)
    assert p.sk_ctas == 0 and p.iters_per_sk_cta == 1 and p.workspace_bytes == 0
    assert p.cta_of(0) == 0                      # no division by zero
    q = P.plan(2, 2, 3, 64, 64, 4, "persistent", "linear", 16)
    assert q.grid == 4 and P.check_plan(q) == []


def test_rejects_bad_pools():
    for bad in (0, -2, -7):
        with pytest.raises(ValueError):
            P.plan(1, 1, 4, 64, 64, 4, "dp_sk", "linear", bad)
    with pytest.raises(ValueError):
        P.plan(1, 1, 4, 64, 64, 4, "split_k", "linear", 4)
    with pytest.raises(ValueError):
        P.plan(1, 1, 4, 64, 64, 4, "dp_sk", "fancy", 4)


@pytest.mark.parametrize("mode", ["dp_sk", "persistent", "dp"])
def test_bruteforce_invariants(mode):
    n = 0
    for T in range(1, 25):
        tiles_m = 1 if T % 2 else 2
        tiles_n = T // tiles_m
        for ipt in range(1, 21):
            for pool in range(1, 41):
                if mode != "dp_sk" and (pool % 3):
                    continue
                p = P.plan(tiles_m, tiles_n, ipt, 32, 32, 4, mode, "linear", pool)
                assert P.check_plan(p) == [], (T, ipt, pool)
                n += 1
    assert n > 1000


def test_checker_catches_planted_mistakes():
    p = P.plan(1, 3, 10, 32, 32, 4, "dp_sk", "linear", 4)
    assert P.check_plan(p) == []

    class OffByOne(P.Plan):
        def sk_range(self, b):
            s, e = super().sk_range(b)
            return s, e + (1 if b == 1 else 0)

    bad = OffByOne(**p.__dict__)
    assert "a MAC iteration is not covered exactly once" in P.check_plan(bad)

    class WrongInverse(P.Plan):
        def cta_of(self, it):
            return it // (self.iters_per_sk_cta + 1)

    assert "inverse map disagrees with the ranges" in P.check_plan(WrongInverse(**p.__dict__))
    # an unclamped all-DP divisor is flagged
    q = P.plan(2, 2, 5, 32, 32, 4, "dp_sk", "linear", 4)
    assert q.sk_ctas == 0
    assert P.check_plan(replace(q, iters_per_sk_cta=0)) != []


@pytest.mark.parametrize("reduction", ["linear", "tree"])
def test_waits_target_higher_ctas_and_resident_pool_completes(reduction):
    for T in (1, 3, 5, 7, 12):
        for ipt in (1, 3, 8, 13):
            for pool in (2, 3, 5, 8, 11):
                for mode in ("dp_sk", "persistent"):
                    p = P.plan(1, T, ipt, 32, 32, 4, mode, reduction, pool)
                    assert S.waits_target_higher(p)
                    assert S.completes(p, max(p.sk_ctas, 1))
                    cap = S.min_capacity(p)
                    assert cap is not None and cap <= max(p.sk_ctas, 1)


def test_simulator_reports_stall_below_capacity():
    # One tile, four CTAs, linear: the owner (CTA 0) waits on CTAs 1..3 while
    # holding its slot, so a single resident CTA cannot finish.
    p = P.plan(1, 1, 8, 32, 32, 4, "dp_sk", "linear", 4)
    assert not S.completes(p, 1)
    assert S.completes(p, 2)
    assert S.min_capacity(p) == 2
    # Tree on the same plan: CTA 2 waits on 3 and publishes, CTA 0 waits on
    # 1 then 2.
    t = P.plan(1, 1, 8, 32, 32, 4, "dp_sk", "tree", 4)
    assert S.events(t, 0) == [("wait", 1), ("wait", 2)]
    assert S.events(t, 1) == [("pub", 1)]
    assert S.events(t, 2) == [("wait", 3), ("pub", 2)]
    assert S.events(t, 3) == [("pub", 3)]


@pytest.mark.parametrize("reduction", ["linear", "tree"])
def test_persistent_early_segments_only_wait_on_earlier_running_segments(reduction):
    # Persistent launches run a CTA's first segment before its DP tiles when
    # that segment continues a tile begun by a lower CTA (a non-owner), and
    # its other segments after them.  Every wait of such an early segment
    # must target a segment that also runs early in its own CTA -- the first
    # segment, in the same tile, of a higher CTA that is a non-owner too --
    # so the early phase completes on its own and no CTA waits on work
    # queued behind a DP tile.  The waits are derived here from the tile's
    # contributor list (linear: none; tree: the binomial partners before the
    # round in which the position publishes) and must also be the first
    # events of the CTA in the dispatch model.
    n = 0
    for T in range(1, 14):
        for ipt in (1, 2, 3, 5, 8, 13, 20):
            for pool in (2, 3, 4, 5, 7, 8, 11, 16, 23):
                p = P.plan(1, T, ipt, 32, 32, 4, "persistent", reduction, pool)
                for b in range(p.sk_ctas):
                    segs = p.segments(b)
                    if not segs or segs[0][3]:       # starts its tile: not early
                        continue
                    contrib = p.contributors(segs[0][0] - p.dp_tiles)
                    pos = contrib.index(b)
                    assert pos > 0
                    partners = []
                    s = 1
                    while reduction == "tree" and s < len(contrib):
                        if pos % (2 * s) == s:
                            break
                        if pos + s < len(contrib):
                            partners.append(contrib[pos + s])
                        s *= 2
                    expect = [("wait", c) for c in partners] + [("pub", b)]
                    assert S.events(p, b)[:len(expect)] == expect
                    for c in partners:
                        cs = p.segments(c)
                        assert c > b and cs[0][0] == segs[0][0] and not cs[0][3]
                        n += 1
    if reduction == "tree":
        assert n > 100


def test_scatter_plan_needs_whole_slices():
    # 3 tiles x 12 iterations over 3 x 4 CTAs: 4 slices of 3 iterations each.
    p = P.plan(1, 3, 12, 32, 32, 4, "dp_sk", "scatter", 12)
    assert p.whole_slices() and p.iters_per_sk_cta == 3
    # same workspace as linear / tree
    t = P.plan(1, 3, 12, 32, 32, 4, "dp_sk", "tree", 12)
    assert (p.flags_bytes, p.partials_bytes, p.workspace_bytes) == \
        (t.flags_bytes, t.partials_bytes, t.workspace_bytes)
    for pool in (5, 7, 8, 11):   # ranges that straddle tiles or split unevenly
        assert not P.plan(1, 3, 12, 32, 32, 4, "dp_sk", "tree", pool).whole_slices()
        with pytest.raises(ValueError):
            P.plan(1, 3, 12, 32, 32, 4, "dp_sk", "scatter", pool)
    # all-DP plans have nothing to reduce and are accepted
    assert P.plan(1, 3, 12, 32, 32, 4, "dp", "scatter", 3).sk_ctas == 0
    assert P.default_pool("scatter", 256, 2) == 256


def test_scatter_parts_partition_every_tile():
    # Under the scatter fix-up each tile's units are cut into the S parts its
    # contributors write: together they cover the tile once, in contributor
    # order, and each part sums exactly the tile's contributors (as the
    # partitioner's own inverse map finds them).
    n = 0
    for T in (1, 2, 3, 5, 9, 18):
        for ipt in (2, 6, 12, 28, 1568):
            for S in range(2, 29):
                if ipt % S:
                    continue
                p = P.plan(1, T, ipt, 32, 32, 4, "dp_sk", "scatter", T * S)
                assert p.whole_slices()
                for units in (256, 4096, 16384, 1000):
                    for t in range(T):
                        contrib = p.contributors(t)
                        assert len(contrib) == S
                        cover = []
                        for b in contrib:
                            lo, hi, who = p.scatter_part(b, units)
                            assert who == contrib
                            cover += list(range(lo, hi))
                        assert cover == list(range(units)), (T, ipt, S, units, t)
                n += 1
    assert n > 100


def test_scatter_needs_the_whole_group_resident():
    # Every contributor waits on all the others, lower ids included: the
    # group of n must be resident at once, and is enough in block order.
    for T, ipt, n in [(1, 8, 4), (3, 12, 4), (2, 28, 7), (5, 6, 3)]:
        p = P.plan(1, T, ipt, 32, 32, 4, "dp_sk", "scatter", T * n)
        assert not S.waits_target_higher(p)
        assert S.min_capacity(p) == n
        assert not S.completes(p, n - 1)
        assert S.completes(p, T * n)
        assert S.events(p, 1)[0] == ("pub", 1)
        assert sorted(c for k, c in S.events(p, 1) if k == "wait") == \
            [c for c in range(n) if c != 1]


def test_dgrad_phases_by_brute_force():
    # Every input pixel lies in exactly one phase; a phase's taps are
    # exactly the taps whose shifted position is a multiple of the stride,
    # which include every tap that reaches an output pixel of that pixel.
    for (H, W, R, S, sh, sw, ph, pw) in [(9, 9, 3, 3, 2, 2, 1, 1), (28, 28, 3, 3, 2, 2, 1, 1),
                                         (11, 7, 5, 5, 2, 1, 2, 2), (10, 13, 3, 2, 3, 2, 0, 1),
                                         (5, 6, 1, 1, 2, 2, 0, 0), (8, 8, 3, 3, 1, 1, 1, 1),
                                         (3, 4, 4, 4, 4, 3, 1, 2)]:
        ho = (H + 2 * ph - R) // sh + 1
        wo = (W + 2 * pw - S) // sw + 1
        phases = P.dgrad_phases(H, W, R, S, sh, sw, ph, pw)
        assert len(phases) == sh * sw
        owner = {}
        for (a, b, h0, w0, hc, wc, rc, sc) in phases:
            taps = {(a + sh * i, b + sw * j) for i in range(rc) for j in range(sc)}
            assert all(r < R and s < S for (r, s) in taps)
            for i in range(hc):
                for j in range(wc):
                    h, w = h0 + sh * i, w0 + sw * j
                    assert 0 <= h < H and 0 <= w < W and (h, w) not in owner
                    owner[(h, w)] = (a, b)
                    exact = {(r, s) for r in range(R) for s in range(S)
                             if (h + ph - r) % sh == 0 and (w + pw - s) % sw == 0}
                    assert exact == taps
                    reach = {(r, s) for (r, s) in exact
                             if 0 <= (h + ph - r) // sh < ho and 0 <= (w + pw - s) // sw < wo}
                    assert reach <= taps
        assert len(owner) == H * W
