"""Host-side mirror of the overlapped forward's ticket tables (the table
construction of queue_build_kernel in csrc/moe_queue.hip), and the schedule
properties its no-deadlock argument rests on.  Test infrastructure.

The overlapped forward runs dispatch items, W1 + SwiGLU tiles and W2 tiles of
one layer in one launch.  Workgroup b takes one ticket from queue b % 8 and
runs that one item: a dispatch item copies 64 x_perm rows and raises its flag;
a W1 tile waits for the flags of the dispatch items holding its rows; a W2
tile waits until every W1 tile of its m-tile is done.  The schedule cannot
deadlock whether or not all workgroups are resident if every wait targets an
item of the waiting item's own queue with a smaller ticket: tickets of a queue
are handed out in increasing order, so such an item was taken by a workgroup
that is already running, and dispatch items never wait.

`build` computes what the kernel writes for a routing (per-queue row bounds R,
dispatch-item bases CB, ticket-table bases BASE and the table); `check` tests
that schedule; `build_looped_variant` is the table construction of the earlier
looped persistent variant (one workgroup per CU cycling over tickets), for the
same check.
"""
from __future__ import annotations

import numpy as np

XCDS = 8
CHUNK_ROWS = 64   # x_perm rows per dispatch item
LEAD = 160        # dispatch items placed ahead of the W1 tiles needing them
KIND_CHUNK, KIND_W1, KIND_W2 = 0, 1, 2


def part(n: int, x: int) -> int:
    return n * x // XCDS


def tile_prefix(counts, rows=256):
    """[E+1] prefix sum of ceil(count / rows), as the routing step writes it."""
    return np.concatenate([[0], np.cumsum(-(-np.asarray(counts, np.int64) // rows))]).astype(np.int64)


def expert_of(tile256, mt):
    """Largest e in [0, E) with tile256[e] <= mt."""
    E = len(tile256) - 1
    lo, hi = 0, E
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if tile256[mid] <= mt:
            lo = mid
        else:
            hi = mid
    return lo


def m_tile_rows(offsets, tile256, mt):
    """First x_perm row and row count of global 256-row m-tile mt."""
    e = expert_of(tile256, mt)
    e0, ne = int(offsets[e]), int(offsets[e + 1] - offsets[e])
    m0 = (mt - int(tile256[e])) * 256
    return e0 + m0, min(256, ne - m0)


def capacities(N: int, E: int, ntn2: int, ntn3: int):
    """Table capacity and workgroups per queue that the host launches."""
    mt_cap = (N + E * 255) // 256
    nc_cap = -(-N // CHUNK_ROWS) + XCDS
    per_xcd = -(-mt_cap // XCDS) * (-(-256 // CHUNK_ROWS) + ntn2 + ntn3) + 1
    return nc_cap + mt_cap * (ntn2 + ntn3), per_xcd


def build(offsets, ntn2: int, ntn3: int):
    """Tables for routing offsets [E+1] (offsets[E] = valid pairs)."""
    offsets = np.asarray(offsets, np.int64)
    E = len(offsets) - 1
    tile256 = tile_prefix(np.diff(offsets))
    MT, nvalid = int(tile256[E]), int(offsets[E])

    def first_row(mt):
        return nvalid if mt >= MT else m_tile_rows(offsets, tile256, mt)[0]

    R = [first_row(part(MT, x)) for x in range(XCDS + 1)]
    CB, BASE = [0], [0]
    for x in range(XCDS):
        nc = -(-(R[x + 1] - R[x]) // CHUNK_ROWS)
        nm = part(MT, x + 1) - part(MT, x)
        CB.append(CB[x] + nc)
        BASE.append(BASE[x] + nc + nm * (ntn2 + ntn3))
    G2, G3, NC = MT * ntn2, MT * ntn3, CB[XCDS]

    def xcd_of_mtile(mt):
        x = 0
        while x + 1 < XCDS and part(MT, x + 1) <= mt:
            x += 1
        return x

    def before(g, x):
        first, n = m_tile_rows(offsets, tile256, g // ntn2)
        last = first + n - 1
        return min((last - R[x]) // CHUNK_ROWS + 1 + LEAD, CB[x + 1] - CB[x])

    table = np.full(BASE[XCDS], -1, np.int64)
    writes = np.zeros(BASE[XCDS], np.int64)

    def put(pos, val):
        table[pos] = val
        writes[pos] += 1

    for i in range(G2):
        x = xcd_of_mtile(i // ntn2)
        put(BASE[x] + (i - part(MT, x) * ntn2) + before(i, x), (KIND_W1 << 28) | i)
    for i in range(NC):
        x = 0
        while x + 1 < XCDS and CB[x + 1] <= i:
            x += 1
        cl = i - CB[x]
        lo, hi = part(MT, x) * ntn2, part(MT, x + 1) * ntn2   # first W1 tile placed after it
        g0 = lo
        while lo < hi:
            mid = (lo + hi) // 2
            if before(mid, x) <= cl:
                lo = mid + 1
            else:
                hi = mid
        put(BASE[x] + cl + (lo - g0), (KIND_CHUNK << 28) | i)
    for i in range(G3):
        x = xcd_of_mtile(i // ntn3)
        nm = part(MT, x + 1) - part(MT, x)
        put(BASE[x] + (CB[x + 1] - CB[x]) + nm * ntn2 + (i - part(MT, x) * ntn3), (KIND_W2 << 28) | i)
    return dict(R=R, CB=CB, BASE=BASE, table=table, writes=writes, MT=MT, nvalid=nvalid,
                tile256=tile256, offsets=offsets, ntn2=ntn2, ntn3=ntn3, G2=G2, G3=G3, NC=NC)


def check(t, N: int):
    """Raises AssertionError unless the schedule t (from `build`) has every
    property the overlapped forward relies on; N = T * K routed pairs."""
    R, CB, BASE, table = t["R"], t["CB"], t["BASE"], t["table"]
    offsets, tile256, ntn2, ntn3 = t["offsets"], t["tile256"], t["ntn2"], t["ntn3"]
    MT, G2, G3, NC = t["MT"], t["G2"], t["G3"], t["NC"]
    E = len(offsets) - 1
    # every slot written once; every item in exactly one slot
    assert np.all(t["writes"] == 1), "a table slot written twice or never"
    want = sorted([(KIND_CHUNK << 28) | i for i in range(NC)] + [(KIND_W1 << 28) | i for i in range(G2)]
                  + [(KIND_W2 << 28) | i for i in range(G3)])
    assert sorted(table.tolist()) == want, "the tickets are not a bijection onto the items"
    # queue and ticket of every item
    where = {}
    for x in range(XCDS):
        for tk in range(BASE[x + 1] - BASE[x]):
            where[int(table[BASE[x] + tk])] = (x, tk)
    # the dispatch items of queue x copy exactly rows [R[x], R[x+1]); together [0, nvalid)
    assert R[0] == 0 and R[XCDS] == t["nvalid"] and all(R[x] <= R[x + 1] for x in range(XCDS))
    for i in range(NC):
        x, _ = where[(KIND_CHUNK << 28) | i]
        assert CB[x] <= i < CB[x + 1]
    for g in range(G2):
        x, tk = where[(KIND_W1 << 28) | g]
        first, n = m_tile_rows(offsets, tile256, g // ntn2)
        assert n >= 1 and R[x] <= first and first + n <= R[x + 1], "W1 tile rows outside its queue"
        for ch in range((first - R[x]) // CHUNK_ROWS, (first + n - 1 - R[x]) // CHUNK_ROWS + 1):
            assert CB[x] + ch < CB[x + 1], "W1 tile waits on another queue's dispatch item"
            xi, ti = where[(KIND_CHUNK << 28) | (CB[x] + ch)]
            assert xi == x and ti < tk, "W1 tile waits on a later or foreign ticket"
    for g in range(G3):
        x, tk = where[(KIND_W2 << 28) | g]
        mt = g // ntn3
        for nt in range(ntn2):
            xi, ti = where[(KIND_W1 << 28) | (mt * ntn2 + nt)]
            assert xi == x and ti < tk, "W2 tile waits on a later or foreign ticket"
    # capacities: the table fits its region and every ticket has a workgroup
    cap, per_xcd = capacities(N, E, ntn2, ntn3)
    assert BASE[XCDS] <= cap
    assert max(BASE[x + 1] - BASE[x] for x in range(XCDS)) <= per_xcd


def build_looped_variant(offsets, N: int, ntn2: int, ntn3: int):
    """The earlier looped persistent variant's tables (256-row dispatch items
    over the whole pair range, split into queues by item index; W1 and W2 tiles
    split into queues by flat tile index; items placed 2 ahead).  Returns its
    table, queue bases, the (queue, ticket) of every item, and its waits: for
    each (queue, ticket) the (queue, ticket) pairs that item waited on."""
    offsets = np.asarray(offsets, np.int64)
    E = len(offsets) - 1
    tile256 = tile_prefix(np.diff(offsets))
    MT = int(tile256[E])
    chunk, lead = 256, 2
    NC = -(-N // chunk)
    G2, G3 = MT * ntn2, MT * ntn3

    def base(x):
        return part(NC, x) + part(G2, x) + part(G3, x)

    def need(g):
        first, n = m_tile_rows(offsets, tile256, g // ntn2)
        return (first + n - 1) // chunk

    def before(g, x):
        n = part(NC, x + 1) - part(NC, x)
        return min(max(need(g) + 1 + lead - part(NC, x), 0), n)

    def queue_of(i, n):
        x = 0
        while x + 1 < XCDS and part(n, x + 1) <= i:
            x += 1
        return x

    table = np.full(base(XCDS), -1, np.int64)
    for i in range(G2):
        x = queue_of(i, G2)
        table[base(x) + (i - part(G2, x)) + before(i, x)] = (KIND_W1 << 28) | i
    for i in range(NC):
        x = queue_of(i, NC)
        cl = i - part(NC, x)
        lo, hi = part(G2, x), part(G2, x + 1)
        while lo < hi:
            mid = (lo + hi) // 2
            if before(mid, x) <= cl:
                lo = mid + 1
            else:
                hi = mid
        table[base(x) + cl + (lo - part(G2, x))] = (KIND_CHUNK << 28) | i
    for i in range(G3):
        x = queue_of(i, G3)
        first = base(x) + (part(NC, x + 1) - part(NC, x)) + (part(G2, x + 1) - part(G2, x))
        table[first + (i - part(G3, x))] = (KIND_W2 << 28) | i
    where = {}
    for x in range(XCDS):
        for tk in range(base(x + 1) - base(x)):
            where[int(table[base(x) + tk])] = (x, tk)
    waits = {}
    for g in range(G2):
        first, n = m_tile_rows(offsets, tile256, g // ntn2)
        waits[where[(KIND_W1 << 28) | g]] = [where[(KIND_CHUNK << 28) | ch]
                                             for ch in range(first // chunk, (first + n - 1) // chunk + 1)]
    for g in range(G3):
        mt = g // ntn3
        waits[where[(KIND_W2 << 28) | g]] = [where[(KIND_W1 << 28) | (mt * ntn2 + nt)]
                                             for nt in range(ntn2)]
    return dict(table=table, where=where, waits=waits, base=[base(x) for x in range(XCDS + 1)])


CTRL_TICKETS, CTRL_TOTALS, CTRL_BASES, CTRL_ROWS, CTRL_CHUNK_BASE, CTRL_WORDS = 0, 8, 16, 24, 33, 42


def region_offsets(N: int, E: int, ntn2: int, ntn3: int):
    """Byte offsets of the control words, flags, W1-done counters and ticket
    table inside the queue region of the scratch (MOE_VIEW_QUEUE)."""
    def a256(v):
        return (v + 255) // 256 * 256
    mt_cap = (N + E * 255) // 256
    nc_cap = -(-N // CHUNK_ROWS) + XCDS
    ctrl = 0
    flags = a256(CTRL_WORDS * 4)
    f2done = flags + a256(nc_cap * 4)
    table = f2done + a256(mt_cap * 4)
    return dict(ctrl=ctrl, flags=flags, f2done=f2done, table=table,
                table_words=nc_cap + mt_cap * (ntn2 + ntn3))
