"""Data-parallel + stream-K partition of a tiled GEMM (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Written step by step from rocm-libraries PR #13151 ("feat(rocke): stream-K for
implicit-GEMM conv wgrad"): the Partitioner bullet of Technical Details, the
commit that adds the iteration partitioner (whole waves of output tiles run
data-parallel, the remainder's MAC iterations are spread as contiguous,
balanced ranges over the pool, a range may straddle tiles, the plan is
resolved once on the host), review item 1 (the iterations-per-CTA clamp and
the inverse map from an iteration to its CTA), review item 2 and the verdict
table (one flag per CTA and wave), the commit sizing the default pool (one
CTA per CU for linear / tree, four per CU for atomic / workspace), and the
bot review comment on the automatic selection (a one-tile remainder smaller
than the pool leaves no stream-K CTAs).

Vocabulary: a *MAC iteration* is one TM x TN x TK block of multiply-adds of one
output tile; a tile has ``ipt = ceil(Kred / TK)`` of them.  ``P`` is the CTA
pool.  Readings where the page leaves a step open:

* DP/SK split: ``dp_tiles = (T // P) * P`` -- whole waves of the pool;
* if the remainder has fewer MAC iterations than the pool the plan is all-DP;
* DP tiles are the first ``dp_tiles`` tile ids, the stream-K tiles the rest;
* the first ``extra`` stream-K CTAs take one iteration more than the others;
* a tile's owner is the CTA that runs its first iteration;
* ``dp_sk`` launches the stream-K CTAs first (block ids ``[0, sk_ctas)``),
  then one CTA per DP tile; ``persistent`` launches the pool, each CTA running
  its stream-K range and then DP tiles ``b, b + grid, ...``.
"""

from dataclasses import dataclass

MODES = ("dp", "dp_sk", "persistent")
# "scatter" is not one of the page's four fix-ups: a one-round deterministic
# reduce-scatter for partitions whose stream-K CTAs each hold one whole slice
# of one tile (every contributor publishes its partial; contributor k of the
# tile's S sums the k-th of S equal parts over all S partials in contributor
# order).  It waits on other CTAs like linear / tree and uses their workspace.
REDUCTIONS = ("linear", "tree", "atomic", "workspace", "scatter")
HANDOFF = ("linear", "tree", "scatter")


def ceil_div(a, b):
    return -(-a // b)


def default_pool(reduction, num_cus, resident_per_cu):
    """Pool used for ``ctas = -1``: one CTA per CU for the reductions that wait
    on other CTAs (linear, tree, scatter), four per CU for those that never wait
    (atomic, workspace); never more than the device keeps resident."""
    if reduction not in REDUCTIONS:
        raise ValueError("unknown reduction")
    if num_cus <= 0 or resident_per_cu <= 0:
        raise ValueError("device has no resident capacity")
    per_cu = 1 if reduction in HANDOFF else 4
    return num_cus * min(per_cu, resident_per_cu)


@dataclass(frozen=True)
class Plan:
    tiles_m: int
    tiles_n: int
    tiles: int
    iters_per_tile: int
    pool: int
    mode: str
    reduction: str
    dp_tiles: int
    sk_tiles: int
    sk_ctas: int
    sk_iters: int
    iters_per_sk_cta: int      # clamped to >= 1
    extra_iters: int
    grid: int
    max_contrib: int
    linear_partners: int
    tree_rounds: int
    n_waves: int
    flags_bytes: int
    partials_bytes: int
    workspace_bytes: int       # total bytes the caller must supply

    def whole_slices(self):
        """Every stream-K CTA runs exactly one slice of one tile: the tile's
        iterations split into S = ipt / ipc equal slices, one CTA each."""
        ipc, ipt = self.iters_per_sk_cta, self.iters_per_tile
        return (self.sk_ctas > 0 and self.extra_iters == 0 and ipt % ipc == 0
                and self.sk_ctas == self.sk_tiles * (ipt // ipc))

    def scatter_part(self, b, units):
        """Units ``[lo, hi)`` of a tile's ``units`` that stream-K CTA b sums
        and writes under the scatter fix-up, with the contributors it sums in
        order: the k-th of S equal parts for contributor k = b mod S."""
        S = self.iters_per_tile // self.iters_per_sk_cta
        c0, k = (b // S) * S, b % S
        return k * units // S, (k + 1) * units // S, list(range(c0, c0 + S))

    # -- the per-CTA view --------------------------------------------------
    def sk_range(self, b):
        """Global stream-K iterations ``[start, end)`` of stream-K CTA b."""
        ipc, extra = self.iters_per_sk_cta, self.extra_iters
        start = b * ipc + min(b, extra)
        end = start + ipc + (1 if b < extra else 0)
        return start, end

    def cta_of(self, it):
        """Stream-K CTA that runs global stream-K iteration ``it``."""
        ipc, extra = self.iters_per_sk_cta, self.extra_iters
        boundary = extra * (ipc + 1)
        if it < boundary:
            return it // (ipc + 1)
        return extra + (it - boundary) // ipc

    def contributors(self, sk_tile):
        """CTAs that run part of stream-K tile ``sk_tile`` (0-based among the
        stream-K tiles), in increasing order; the first is the owner."""
        first = sk_tile * self.iters_per_tile
        last = first + self.iters_per_tile - 1
        return list(range(self.cta_of(first), self.cta_of(last) + 1))

    def segments(self, b):
        """Tile segments of stream-K CTA b in the order it runs them:
        ``(tile_id, k_begin, k_end, started, ended)`` with k in MAC
        iterations of that tile."""
        start, end = self.sk_range(b)
        out = []
        it = start
        ipt = self.iters_per_tile
        while it < end:
            t = it // ipt
            seg_end = min(end, (t + 1) * ipt)
            k0, k1 = it - t * ipt, seg_end - t * ipt
            out.append((self.dp_tiles + t, k0, k1, k0 == 0, k1 == ipt))
            it = seg_end
        return out

    def dp_tiles_of(self, block):
        """DP tile ids that grid block ``block`` runs."""
        if self.mode == "dp":
            return [block]
        if self.mode == "dp_sk":
            return [block - self.sk_ctas] if block >= self.sk_ctas else []
        return list(range(block, self.dp_tiles, self.grid))


def plan(tiles_m, tiles_n, iters_per_tile, tm, tn, n_waves,
         mode, reduction, ctas, num_cus=None, resident_per_cu=None):
    """Resolve the launch plan of a GEMM with ``tiles_m x tiles_n`` output
    tiles of ``tm x tn`` and ``iters_per_tile`` MAC iterations each."""
    if mode not in MODES:
        raise ValueError("unknown mode")
    if reduction not in REDUCTIONS:
        raise ValueError("unknown reduction")
    if tiles_m <= 0 or tiles_n <= 0 or iters_per_tile <= 0:
        raise ValueError("empty problem")
    # 1. Tiles.
    T = tiles_m * tiles_n
    ipt = iters_per_tile
    # 2. Pool.
    if ctas == -1:
        if num_cus is None or resident_per_cu is None:
            raise ValueError("default pool needs the device's CU count")
        P = default_pool(reduction, num_cus, resident_per_cu)
    elif ctas > 0:
        P = ctas
    else:
        raise ValueError("streamk ctas must be -1 or positive")
    # 3./4. DP / SK split.
    if mode == "dp":
        dp_tiles, sk_tiles, sk_ctas = T, 0, 0
    else:
        dp_tiles = (T // P) * P
        sk_tiles = T - dp_tiles
        if sk_tiles == 0 or sk_tiles * ipt < P:
            dp_tiles, sk_tiles, sk_ctas = T, 0, 0
        else:
            sk_ctas = P
    sk_iters = sk_tiles * ipt
    # 5. Iterations per stream-K CTA, clamped to at least one.
    ipc_raw = sk_iters // sk_ctas if sk_ctas else 0
    extra = sk_iters % sk_ctas if sk_ctas else 0
    ipc = max(ipc_raw, 1)
    # 9. Grid.
    if mode == "dp":
        grid = T
    elif mode == "dp_sk":
        grid = sk_ctas + dp_tiles
    else:
        grid = P if sk_ctas else min(P, T)
    # 8. Contributors per stream-K tile.
    partial = Plan(tiles_m, tiles_n, T, ipt, P, mode, reduction, dp_tiles,
                   sk_tiles, sk_ctas, sk_iters, ipc, extra, grid, 1, 0, 0,
                   n_waves, 0, 0, 0)
    max_contrib = 1
    for t in range(sk_tiles):
        max_contrib = max(max_contrib, len(partial.contributors(t)))
    tree_rounds = 0
    while (1 << tree_rounds) < max_contrib:
        tree_rounds += 1
    # 10. Bytes.
    flags = partials = ws = 0
    if sk_ctas and reduction in HANDOFF:
        flags = ceil_div(4 * sk_ctas * n_waves, 256) * 256
        partials = sk_ctas * tm * tn * 4
        ws = flags + partials
    elif sk_ctas and reduction == "workspace":
        ws = sk_tiles * tm * tn * 4
    out = Plan(tiles_m, tiles_n, T, ipt, P, mode, reduction, dp_tiles,
               sk_tiles, sk_ctas, sk_iters, ipc, extra, grid, max_contrib,
               max_contrib - 1, tree_rounds, n_waves, flags, partials, ws)
    if reduction == "scatter" and sk_ctas and not out.whole_slices():
        raise ValueError("scatter needs every stream-K CTA to hold one whole slice of one tile")
    return out


def gemm_tiles(M, N, K, tm, tn, tk):
    """(tiles_m, tiles_n, iters_per_tile) of an M x N x K GEMM."""
    return ceil_div(M, tm), ceil_div(N, tn), ceil_div(K, tk)


def wgrad_tiles(N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, groups,
                tm, tn, tk, group_block=0):
    """Implicit-GEMM view of a wgrad: GEMM-M = output channels, folded per
    group (the tile count is per group, so a partial last M tile stays inside
    its group), GEMM-N = Cpg*R*S, reduction = N*Ho*Wo.

    group_block > 0: block-diagonal tiles, each holding group_block whole
    consecutive groups (tm = group_block * Kpg output channels; the columns
    of every row are its own group's Cpg*R*S filter entries), so GEMM-M is
    tiled over all K output channels at once and only the last M tile can
    hold fewer groups."""
    ho = (H + 2 * pad_h - R) // stride_h + 1
    wo = (W + 2 * pad_w - S) // stride_w + 1
    kpg, cpg = K // groups, C // groups
    if group_block:
        if tm != group_block * kpg:
            raise ValueError("a block-diagonal tile holds group_block whole groups")
        tiles_m = ceil_div(groups, group_block)
    else:
        tiles_m = groups * ceil_div(kpg, tm)
    return (tiles_m, ceil_div(cpg * R * S, tn), ceil_div(N * ho * wo, tk))


def _n_tiles(groups, npg, tn, group_block):
    """GEMM-N tiles of a convolution whose N index runs over channels folded
    per group: per group (dense tiles), or group_block whole consecutive
    groups per tile (block-diagonal tiles, tn = group_block * npg)."""
    if group_block:
        if tn != group_block * npg:
            raise ValueError("a block-diagonal tile holds group_block whole groups")
        return ceil_div(groups, group_block)
    return groups * ceil_div(npg, tn)


def fwd_tiles(N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, groups, tm, tn, tk,
              group_block=0):
    """Implicit-GEMM view of a forward convolution: GEMM-M = output pixels
    N*Ho*Wo, GEMM-N = output channels folded per group (the tile count is
    per group, so an N tile never crosses a group; or group_block whole
    groups per block-diagonal tile), reduction = R*S*Cpg per group."""
    ho = (H + 2 * pad_h - R) // stride_h + 1
    wo = (W + 2 * pad_w - S) // stride_w + 1
    kpg, cpg = K // groups, C // groups
    return (ceil_div(N * ho * wo, tm), _n_tiles(groups, kpg, tn, group_block),
            ceil_div(R * S * cpg, tk))


def dgrad_phases(H, W, R, S, stride_h, stride_w, pad_h, pad_w):
    """Stride phases of the input gradient.  Input row h receives filter row
    r only when h + pad_h - r is a multiple of stride_h, i.e. when r and
    h + pad_h agree modulo stride_h; likewise for columns.  Phase (a, b)
    holds the pixels with (h + pad_h) mod stride_h == a and (w + pad_w) mod
    stride_w == b: rows h0, h0 + stride_h, ... (hc of them), columns w0,
    w0 + stride_w, ... (wc), and its taps are r = a, a + stride_h, ... (rc)
    times s = b, b + stride_w, ... (sc).  Returns one tuple
    (a, b, h0, w0, hc, wc, rc, sc) per phase, row phase major."""
    out = []
    for a in range(stride_h):
        h0 = (a - pad_h) % stride_h
        hc = max(0, ceil_div(H - h0, stride_h))
        rc = max(0, ceil_div(R - a, stride_h))
        for b in range(stride_w):
            w0 = (b - pad_w) % stride_w
            wc = max(0, ceil_div(W - w0, stride_w))
            sc = max(0, ceil_div(S - b, stride_w))
            out.append((a, b, h0, w0, hc, wc, rc, sc))
    return out


def dgrad_tiles(N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, groups, tm, tn, tk,
                group_block=0):
    """Implicit-GEMM view of the input gradient: GEMM-M = input pixels
    N*H*W, GEMM-N = input channels folded per group (or group_block whole
    groups per block-diagonal tile), reduction = R*S*Kpg per group.

    Block-diagonal tiles order GEMM-M by stride phase (dgrad_phases): a tile
    holds pixels of one phase only and reduces over that phase's taps, so
    the M tiles are counted per phase and the iterations per tile are those
    of the phase with the most taps."""
    kpg, cpg = K // groups, C // groups
    if group_block:
        ph = dgrad_phases(H, W, R, S, stride_h, stride_w, pad_h, pad_w)
        tiles_m = sum(ceil_div(N * hc * wc, tm) for (_, _, _, _, hc, wc, _, _) in ph)
        taps = max(rc * sc for (_, _, _, _, _, _, rc, sc) in ph)
        return (tiles_m, _n_tiles(groups, cpg, tn, group_block), max(1, ceil_div(taps * kpg, tk)))
    return (ceil_div(N * H * W, tm), _n_tiles(groups, cpg, tn, group_block),
            ceil_div(R * S * kpg, tk))


def check_plan(p):
    """Brute-force the invariants of a plan over an explicit coverage array.
    Returns a list of violated properties (empty when the plan is sound)."""
    bad = []
    T, ipt = p.tiles, p.iters_per_tile
    cover = [[0] * ipt for _ in range(T)]
    # DP tiles: whole tiles, one CTA each.
    for block in range(p.grid):
        for t in p.dp_tiles_of(block):
            if not (0 <= t < p.dp_tiles):
                bad.append("DP block maps outside the DP tiles")
                continue
            for k in range(ipt):
                cover[t][k] += 1
    # Stream-K ranges.
    prev_end = 0
    lengths = []
    for b in range(p.sk_ctas):
        s, e = p.sk_range(b)
        if s != prev_end:
            bad.append("stream-K ranges not contiguous")
        prev_end = e
        lengths.append(e - s)
        non_owner = 0
        for (t, k0, k1, started, ended) in p.segments(b):
            if not started:
                non_owner += 1
            for k in range(k0, k1):
                cover[t][k] += 1
            for it in range((t - p.dp_tiles) * ipt + k0, (t - p.dp_tiles) * ipt + k1):
                if p.cta_of(it) != b:
                    bad.append("inverse map disagrees with the ranges")
        if non_owner > 1:
            bad.append("more than one non-owner tile in one stream-K CTA")
    if p.sk_ctas and prev_end != p.sk_iters:
        bad.append("stream-K ranges do not end at the last iteration")
    if lengths and max(lengths) - min(lengths) > 1:
        bad.append("stream-K ranges unbalanced")
    if any(c != 1 for row in cover for c in row):
        bad.append("a MAC iteration is not covered exactly once")
    if p.iters_per_sk_cta < 1:
        bad.append("iterations per stream-K CTA below one")
    if p.sk_ctas == 0 and (p.iters_per_sk_cta != 1 or p.extra_iters != 0):
        bad.append("all-DP plan with a non-trivial stream-K split")
    if p.sk_ctas and p.max_contrib > ceil_div(ipt, p.iters_per_sk_cta) + 1:
        bad.append("contributor bound exceeded")
    return bad


# ---------------------------------------------------------------------------
# Automatic launch choice and the split-K comparator (rocm-libraries PR
# #13151: the commit that made stream-K the "auto" default -- stream-K where
# a candidate has few output tiles over a long reduction, the grid-per-tile
# split-K kernel everywhere else, and "auto" for the reduction resolving to
# the workspace fix-up because it never waits and so gets the
# occupancy-sized pool -- and the review follow-up that builds the partition
# the launch will really use and keeps split-K when it has no stream-K
# CTAs).  The pages print no thresholds ("coarse on purpose"); readings:
#
# * few tiles: the tiles leave a ragged data-parallel wave (T mod P != 0)
#   and are fewer than two full waves (T < 2P), so that wave is a large
#   part of the run;
# * long reduction: at least LONG_REDUCTION MAC iterations per tile;
# * split-K cuts every tile into S equal K slices; the default S fills the
#   pool (pool // tiles) but keeps every slice at least LONG_REDUCTION
#   iterations long, since a slice's fp32 partial tile costs a write and a
#   read of about as many bytes as that many iterations' operand tiles; an
#   explicit S is clamped to [1, iters_per_tile] only; S = 1 is plain
#   data-parallel.  It runs on the stream-K engine as dp_sk with a pool of
#   tiles * S CTAs, whose partition has dp_tiles = 0 and gives every CTA
#   one slice (ranges straddle two tiles' slices when S does not divide
#   iters_per_tile).

LONG_REDUCTION = 8


def resolve_launch(tiles, iters_per_tile, mode, reduction, ctas, num_cus=None,
                   resident_per_cu=None):
    """Resolve ``mode in {dp, dp_sk, persistent, splitk, auto}`` and
    ``reduction in {linear, tree, atomic, workspace, auto}`` to the launch
    the planner plans.  Returns ``(mode, reduction, ctas, slices)`` with mode
    one of dp / dp_sk / persistent; ``slices`` is the split-K slice count
    (1 when not split-K)."""
    if reduction == "auto":
        reduction = "workspace"
    if reduction not in REDUCTIONS:
        raise ValueError("unknown reduction")
    if ctas == 0 or ctas < -1:
        raise ValueError("streamk ctas must be -1 or positive")
    T, ipt = tiles, iters_per_tile

    def pool():
        if ctas > 0:
            return ctas
        if num_cus is None or resident_per_cu is None:
            raise ValueError("default pool needs the device's CU count")
        return default_pool(reduction, num_cus, resident_per_cu)

    if mode == "auto":
        P = pool()
        if T % P != 0 and T < 2 * P and ipt >= LONG_REDUCTION:
            # The stream-K partition at this pool has stream-K CTAs unless
            # the remainder tiles hold fewer iterations than the pool.
            if (T - (T // P) * P) * ipt >= P:
                return "dp_sk", reduction, P, 1
        S = min(P // T, ipt // LONG_REDUCTION)  # split-K filling the same pool
    elif mode == "splitk":
        S = min(pool() // T, ipt // LONG_REDUCTION) if ctas == -1 else ctas
    if mode in ("auto", "splitk"):
        S = max(1, min(S, ipt))
        if S == 1:
            return "dp", reduction, T, 1
        return "dp_sk", reduction, T * S, S
    if mode not in MODES:
        raise ValueError("unknown mode")
    return mode, reduction, ctas, 1
