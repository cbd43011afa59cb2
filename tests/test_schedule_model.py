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
A launch that runs two passes interleaves their items phase by phase; the
model checks that every unit keeps its own order inside that interleaving.

Two further models cover how a finished tile reaches its readers: through
the caches (per-CU L1s, per-XCC write-back L2s, memory; stores, L2
write-backs and atomics land asynchronously until waited for), and through
the LDS that a tile's epilogue stages in and the next tile's first copies
overwrite.  Each checks the protocol as built and shows that weakening any
of its steps lets a reader see stale data.
"""

import copy
import itertools
import json

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


def two_pass_order(passes, n_iter):
    """Claim order of a two-pass launch (ns_persistent2): per iteration the
    Gram tiles of the first pass's units (unit-major), then the second
    pass's, then the polynomial tiles of each pass, then the apply tiles of
    each.  passes: (units, ts, tl) per pass; items are (pass, unit, item)."""
    one = [items(ts, tl, n_iter) for _, ts, tl in passes]
    out = []
    for it in range(n_iter):
        for ph in ("G", "P", "A"):
            for k, (units, _, _) in enumerate(passes):
                for u in range(units):
                    out += [(k, u, x) for x in one[k] if x[0] == it and x[1] == ph]
    return out


@pytest.mark.parametrize("passes", [
    [(3, 4, 14), (1, 4, 4)],     # the layer's MLP units with its O projection (16 x 56 and 16 x 16 panels, scaled down)
    [(2, 2, 5), (1, 3, 3)],      # ragged: different small sides
    [(4, 2, 6), (1, 1, 1)],      # a one-tile rider
])
def test_two_pass_order_keeps_each_units_order(passes):
    # Each unit's items keep their own claim order inside the two-pass
    # order, so every dependency still points to an earlier item and every
    # property checked above for one unit's order carries over; items of
    # different units (of either pass) share no buffers.
    n_iter = 3
    order = two_pass_order(passes, n_iter)
    assert len(order) == sum(u * len(items(ts, tl, n_iter)) for u, ts, tl in passes)
    pos = {x: k for k, x in enumerate(order)}
    for k, (units, ts, tl) in enumerate(passes):
        for u in range(units):
            mine = [x for (kk, uu, x) in order if (kk, uu) == (k, u)]
            assert mine == items(ts, tl, n_iter)
            for x in mine:
                for d in deps(x, ts, tl):
                    assert pos[(k, u, d)] < pos[(k, u, x)]


# ------------------------------------------------------------------------
# Publication of a finished tile and its acquisition by a reader, through
# the caches.  Model: each CU has an L1 (a reader keeps lines it loaded);
# each XCC has a write-back L2 that its CUs share; memory is coherent; the
# completion counts are atomics at memory.  A store, the L2 write-back of a
# release and an atomic are issued asynchronously and land at any later
# point, until the issuing wave waits for them (s_waitcnt vmcnt(0)).  An
# agent-scope invalidate (sc1) drops the CU's L1 lines and the clean lines
# of its XCC's L2; the sc0 form does nothing outside thread-group-split mode
# (device probe).  The reader has the tile's old value cached from the
# previous iteration.  Every interleaving is explored; the reader must see
# the new value whenever it has seen the count.

OLD, NEW = "old", "new"


def publish_program(local, wait_store=True, wait_writeback=True):
    """The producer wave's steps after its tile's stores are issued."""
    prog = [("store",)]
    if wait_store:
        prog.append(("wait",))  # every wave's stores complete, then the barrier
    if not local:
        prog.append(("writeback",))  # release at agent scope: buffer_wbl2 sc1
        if wait_writeback:
            prog.append(("wait",))
    prog.append(("count",))
    return prog


def acquire_program(invalidate):
    """The reader: wait for the count, acquire, load the tile."""
    prog = [("see_count",)]
    if invalidate:
        prog += [("invalidate", invalidate), ("wait",)]
    prog.append(("load",))
    return prog


def explore(local, prod, cons):
    """All values the reader can load after seeing the count."""
    px, cx = 0, (0 if local else 1)  # XCC of producer and reader
    progs = {"p": prod, "c": cons}
    init = {
        "mem": {"tile": OLD, "cnt": 0},
        "l2": {0: {}, 1: {}},  # addr -> (value, dirty)
        "l1": {"p": {}, "c": {"tile": OLD}},  # the reader loaded the old tile before
        "pc": {"p": 0, "c": 0},
        "pending": [],  # issued, not landed: (owner, kind, dirty lines of a write-back)
        "got": None,
    }
    init["l2"][cx]["tile"] = (OLD, False)

    def land(s, op):
        _, kind, lines = op
        if kind == "store":  # into the producer's L2 (and its own L1)
            s["l2"][px]["tile"] = (NEW, True)
            s["l1"]["p"]["tile"] = NEW
        elif kind == "writeback":  # the lines that were dirty when it was issued
            for addr, v in lines:
                s["mem"][addr] = v
                if s["l2"][px].get(addr, (None, False))[1]:
                    s["l2"][px][addr] = (s["l2"][px][addr][0], False)
        else:  # the completion count, an atomic at memory
            s["mem"]["cnt"] += 1

    def advance(s, who):
        """`who`'s next step applied to a copy of s, or None if blocked or done."""
        i = s["pc"][who]
        if i >= len(progs[who]):
            return None
        op = progs[who][i]
        if op[0] == "wait" and any(o[0] == who for o in s["pending"]):
            return None
        if op[0] == "see_count" and s["mem"]["cnt"] < 1:
            return None
        t = copy.deepcopy(s)
        t["pc"][who] = i + 1
        if op[0] in ("store", "count"):
            t["pending"].append((who, op[0], ()))
        elif op[0] == "writeback":
            dirty = tuple((a, v) for a, (v, d) in sorted(s["l2"][px].items()) if d)
            t["pending"].append((who, "writeback", dirty))
        elif op[0] == "invalidate" and op[1] == "sc1":
            t["l1"]["c"] = {}
            t["l2"][cx] = {a: v for a, v in s["l2"][cx].items() if v[1]}
        elif op[0] == "load":
            if "tile" in s["l1"]["c"]:
                v = s["l1"]["c"]["tile"]
            elif "tile" in s["l2"][cx]:
                v = s["l2"][cx]["tile"][0]
            else:
                v = s["mem"]["tile"]
                t["l2"][cx]["tile"] = (v, False)
            t["l1"]["c"]["tile"] = v
            t["got"] = v
        return t

    results, seen, stack = set(), set(), [init]
    while stack:
        s = stack.pop()
        k = repr(s)
        if k in seen:
            continue
        seen.add(k)
        if s["got"] is not None:
            results.add(s["got"])
            continue
        nxt = [advance(s, who) for who in ("p", "c")]
        for j, op in enumerate(s["pending"]):
            t = copy.deepcopy(s)
            del t["pending"][j]
            land(t, op)
            nxt.append(t)
        stack += [t for t in nxt if t is not None]
    return results


def test_single_queue_publish_and_acquire_as_built():
    # one queue: producer and reader on different XCCs; stores complete,
    # L2 written back and waited for, then the count; the reader invalidates
    # at agent scope (sc1) after seeing the count
    assert explore(False, publish_program(False), acquire_program("sc1")) == {NEW}


def test_single_queue_without_the_wait_after_the_writeback_reads_stale_data():
    # the count can land before the write-back: the reader, having dropped
    # its caches, fetches the old tile from memory
    got = explore(False, publish_program(False, wait_writeback=False), acquire_program("sc1"))
    assert OLD in got


def test_single_queue_with_an_sc0_acquire_reads_stale_data():
    got = explore(False, publish_program(False), acquire_program("sc0"))
    assert OLD in got


def test_single_queue_counting_before_the_stores_complete_reads_stale_data():
    got = explore(False, publish_program(False, wait_store=False), acquire_program("sc1"))
    assert OLD in got


def test_xcc_local_publish_and_acquire_as_built():
    # one queue per XCC: producer and reader share the L2; no write-back is
    # needed, the reader's agent-scope invalidate drops its stale L1 line
    assert explore(True, publish_program(True), acquire_program("sc1")) == {NEW}


def test_xcc_local_with_an_sc0_acquire_or_none_reads_stale_data():
    assert OLD in explore(True, publish_program(True), acquire_program("sc0"))
    assert OLD in explore(True, publish_program(True), acquire_program(None))


# ------------------------------------------------------------------------
# The LDS a tile's epilogue stages through is the ring the next tile's
# first copies (global -> LDS, asynchronous) write into.  Each wave reads
# back its own staged block (LDS reads complete asynchronously, until
# s_waitcnt lgkmcnt(0)); a copy issued by any wave may land at any later
# point.  As built, the loop head's barrier comes after every wave's
# lgkmcnt(0) wait and before any copy of the next tile is issued.


def lds_explore(waves, wait_lgkm_before_barrier=True, barrier=True, copies_overlap=True):
    """Values the staged reads can return: 'acc' (the epilogue's own data)
    or 'copy' (overwritten by the next tile's copy)."""
    region = {w: ("ring", w) for w in range(waves)}  # staged block of wave w
    copy_target = ("ring", 0) if copies_overlap else ("ring", "free slot")
    init = {"lds": {str(region[w]): "acc" for w in range(waves)}, "pc": [0] * waves,
            "pending": [], "got": []}

    def prog(w):
        p = [("read",)]
        if wait_lgkm_before_barrier:
            p.append(("wait_lgkm",))
        if barrier:
            p.append(("barrier",))
        p.append(("copy",))
        return p

    results = set()
    seen = set()
    stack = [init]
    while stack:
        s = stack.pop()
        k = json.dumps(s, sort_keys=True)
        if k in seen:
            continue
        seen.add(k)
        if all(s["pc"][w] >= len(prog(w)) for w in range(waves)) and not s["pending"]:
            results |= set(s["got"])
            continue
        for w in range(waves):
            p = prog(w)
            i = s["pc"][w]
            if i >= len(p):
                continue
            op = p[i][0]
            t = json.loads(k)
            if op == "read":
                t["pending"].append([w, "read", str(region[w])])
            elif op == "wait_lgkm":
                if any(o[0] == w and o[1] == "read" for o in s["pending"]):
                    continue
            elif op == "barrier":
                if any(s["pc"][v] < i for v in range(waves)):
                    continue  # every wave must reach the barrier
            elif op == "copy":
                t["pending"].append([w, "copy", str(copy_target)])
            t["pc"][w] = i + 1
            stack.append(t)
        for j, o in enumerate(s["pending"]):
            t = json.loads(k)
            t["pending"].pop(j)
            if o[1] == "read":
                t["got"].append(s["lds"][o[2]])
            else:
                t["lds"][o[2]] = "copy"
            stack.append(t)
    return results


def test_next_tile_copies_wait_for_every_staged_read():
    assert lds_explore(2) == {"acc"}


def test_a_barrier_without_the_lds_wait_lets_a_copy_overwrite_a_staged_block():
    # the barrier alone does not complete a wave's LDS reads in flight
    assert "copy" in lds_explore(2, wait_lgkm_before_barrier=False)


def test_copies_under_the_epilogue_need_a_slot_the_staging_does_not_use():
    # starting the next tile's first copies before the barrier is safe only
    # into ring slots that no wave stages its epilogue through
    assert "copy" in lds_explore(2, barrier=False)
    assert lds_explore(2, barrier=False, copies_overlap=False) == {"acc"}
