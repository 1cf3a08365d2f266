"""In-order workgroup dispatch model of the deterministic fix-ups (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

rocm-libraries PR #13151 argues forward progress of the linear and tree
hand-offs from two facts: every wait targets a higher-index CTA, and the
hardware dispatches workgroups in order (review verdict table, first row; the
commit that documents the per-(CTA, wave) flag protocol).  This module checks
both on a plan: it lists, per CTA, the publish and wait events the fix-up
performs in program order, and runs them on a model that keeps at most
``capacity`` CTAs resident and dispatches them in block-id order.

Fix-up semantics modelled (tile contributors ``c_0 < c_1 < ... < c_{n-1}``,
``c_0`` the owner):

* linear -- every non-owner publishes its partial; the owner waits on
  ``c_1 ... c_{n-1}`` in that order;
* tree -- with position ``p = c - c_0`` and stride ``s = 2**r`` for rounds
  ``r = 0, 1, ...``: if ``p % (2s) == 0`` and ``p + s < n`` wait on
  ``c_{p+s}``; if ``p % (2s) == s`` publish and drop out.

* scatter (whole-slice partitions only; not one of the page's fix-ups) --
  every contributor publishes its partial, then waits on every other
  contributor of the tile, lower and higher alike: the tile's contributors
  must all be resident together, so forward progress rests on residency of
  the whole group, not on the order of the waits.

atomic and workspace have no events (nobody waits).
"""

from .partition import Plan


def events(p: Plan, block):
    """Ordered ``("pub", cta)`` / ``("wait", cta)`` events of grid block
    ``block`` (stream-K CTAs are blocks ``[0, sk_ctas)`` in both modes)."""
    ev = []
    if block >= p.sk_ctas or p.reduction not in ("linear", "tree", "scatter"):
        return ev
    for (t, k0, k1, started, ended) in p.segments(block):
        if started and ended:
            continue
        contrib = p.contributors(t - p.dp_tiles)
        n = len(contrib)
        pos = contrib.index(block)
        if p.reduction == "scatter":
            ev.append(("pub", block))
            ev += [("wait", c) for c in contrib if c != block]
        elif p.reduction == "linear":
            if pos == 0:
                ev += [("wait", c) for c in contrib[1:]]
            else:
                ev.append(("pub", block))
        else:
            s = 1
            while s < n:
                if pos % (2 * s) == 0:
                    if pos + s < n:
                        ev.append(("wait", contrib[pos + s]))
                elif pos % (2 * s) == s:
                    ev.append(("pub", block))
                    break
                s *= 2
    return ev


def waits_target_higher(p: Plan):
    """True when every wait of every CTA names a higher block id."""
    for b in range(p.grid):
        for kind, c in events(p, b):
            if kind == "wait" and c <= b:
                return False
    return True


def completes(p: Plan, capacity):
    """Run the in-order dispatch model; True when every CTA finishes."""
    ev = [events(p, b) for b in range(p.grid)]
    pc = [0] * p.grid            # next event index per CTA
    published = set()
    running = []
    next_block = 0
    done = 0
    while done < p.grid:
        while next_block < p.grid and len(running) < capacity:
            running.append(next_block)
            next_block += 1
        progressed = False
        for b in list(running):
            while pc[b] < len(ev[b]):
                kind, c = ev[b][pc[b]]
                if kind == "pub":
                    published.add(c)
                elif c not in published:
                    break
                pc[b] += 1
                progressed = True
            if pc[b] == len(ev[b]):
                running.remove(b)
                done += 1
                progressed = True
        if not progressed:
            return False
    return True


def min_capacity(p: Plan):
    """Smallest resident capacity with which the plan completes."""
    lo, hi = 1, max(p.grid, 1)
    if not completes(p, hi):
        return None
    while lo < hi:
        mid = (lo + hi) // 2
        if completes(p, mid):
            hi = mid
        else:
            lo = mid + 1
    return lo
