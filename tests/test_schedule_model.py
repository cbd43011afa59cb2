"""A model of the persistent schedule's dependency rules, checked on the CPU.

Per iteration the schedule runs, for one unit, the Gram tiles (r, c) with
r <= c over the ts tile panels of the small side, then the polynomial tiles
(same grid), then the apply tiles (i, j): small-side panel i, large-side
panel j.  A tile waits only for the panels it reads:
  Gram (r, c) of iteration it > 0: the apply tiles of panels r and c of
      iteration it - 1 (count it * tl per panel);
  polynomial (r, c): the Gram tiles touching panels r and c;
  apply (i, j): the polynomial tiles touching panel i.
The model checks, for small grids and several iterations, that every
dependency points to an earlier item in claim order (so the schedule makes
progress) and that every write to a buffer that is rewritten each iteration
(A, B' and the two iterates) comes after every read of the same region, and
every read after the write it needs, directly or through other dependencies.
"""

import itertools

import pytest


def items(ts, tl, n_iter):
    """Claim order of one unit's items: (iteration, phase, tile)."""
    sym = [(r, c) for r in range(ts) for c in range(r, ts)]
    app = [(i, j) for i in range(ts) for j in range(tl)]
    out = []
    for it in range(n_iter):
        out += [(it, "G", t) for t in sym]
        out += [(it, "P", t) for t in sym]
        out += [(it, "A", t) for t in app]
    return out


def touches(tile, p):
    return p in tile


def deps(item, ts, tl):
    """The items one item waits for, by the rules above."""
    it, ph, t = item
    if ph == "G":
        if it == 0:
            return []
        return [(it - 1, "A", (i, j)) for i in set(t) for j in range(tl)]
    sym = [(r, c) for r in range(ts) for c in range(r, ts)]
    if ph == "P":
        return [(it, "G", s) for s in sym if touches(s, t[0]) or touches(s, t[1])]
    return [(it, "P", s) for s in sym if touches(s, t[0])]


def closure(all_items, ts, tl):
    """Every item's transitive dependencies."""
    memo = {}
    for x in all_items:  # claim order: dependencies are computed first
        acc = set()
        for d in deps(x, ts, tl):
            acc.add(d)
            acc |= memo[d]
        memo[x] = acc
    return memo


def regions(item, ts, tl):
    """(buffer, region) pairs the item writes and reads.  Buffers: 'A', 'B'
    (one each, rewritten every iteration) and 'X0', 'X1' (the iterate of
    iteration it lives in X{it % 2}); regions are tiles."""
    it, ph, t = item
    x_in, x_out = f"X{it % 2}", f"X{(it + 1) % 2}"
    w, r = set(), set()
    if ph == "G":
        a, b = t
        w |= {("A", (a, b)), ("A", (b, a))}  # the tile and its mirror
        r |= {(x_in, (p, j)) for p in (a, b) for j in range(tl)}  # iterate panels a, b
    elif ph == "P":
        a, b = t
        w |= {("B", (a, b)), ("B", (b, a))}
        r |= {("A", (p, k)) for p in (a, b) for k in range(ts)}  # A row panels a, b
    else:
        i, j = t
        w.add((x_out, (i, j)))
        r |= {("B", (i, k)) for k in range(ts)}  # B' row panel i
        r |= {(x_in, (k, j)) for k in range(ts)}  # the iterate's column panel j
    return w, r


@pytest.mark.parametrize("ts,tl", [(1, 1), (1, 3), (2, 2), (2, 5), (3, 3), (3, 4), (4, 6)])
def test_dependencies_point_back_and_order_every_access(ts, tl):
    n_iter = 4
    order = items(ts, tl, n_iter)
    pos = {x: k for k, x in enumerate(order)}
    for x in order:
        for d in deps(x, ts, tl):
            assert pos[d] < pos[x], (x, d)
    before = closure(order, ts, tl)

    def ordered(first, second):
        return first in before[second]

    acc = {x: regions(x, ts, tl) for x in order}
    for x, y in itertools.combinations(order, 2):  # x claimed before y
        wx, rx = acc[x]
        wy, ry = acc[y]
        # a later write to what x read or wrote must wait for x
        if wy & (rx | wx):
            assert ordered(x, y), ("write after access", x, y, sorted(wy & (rx | wx)))
        # a later read of what x wrote must wait for x, unless another
        # write to the region comes in between (then it needs that one)
        for reg in ry & wx:
            last = max((z for z in order if pos[z] < pos[y] and reg in acc[z][0]), key=pos.get)
            assert ordered(last, y), ("read after write", last, y, reg)


@pytest.mark.parametrize("ts,tl", [(1, 2), (2, 3), (3, 2), (4, 4)])
def test_counts_cannot_run_ahead(ts, tl):
    # The kernel keeps one cumulative count per product and panel and waits
    # for count >= (iterations so far) * (tiles per panel per iteration).
    # That equals waiting for the exact tiles above only if no tile can
    # finish before every tile of the same product and panel of the
    # previous iteration: each such tile is among its dependencies.
    order = items(ts, tl, 4)
    before = closure(order, ts, tl)

    def panels(x):
        return set(x[2]) if x[1] != "A" else {x[2][0]}

    for x in order:
        it, ph, _ = x
        if it == 0:
            continue
        for y in order:
            if y[0] == it - 1 and y[1] == ph and panels(x) & panels(y):
                assert y in before[x], (x, y)


def test_iteration_zero_reads_no_earlier_item():
    # the first Gram reads N / nu, written before the launch
    assert deps((0, "G", (0, 1)), 2, 3) == []
