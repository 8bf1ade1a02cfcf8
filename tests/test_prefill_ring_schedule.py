"""A CPU model of the matrix-core prefill's tile schedule for workgroups of one
head (256 consecutive rows), whose two halves walk the raw window apart.

The model restates the kernel's index rules: the union of the rows' raw
windows is tiles 0 .. n_rt-1 (64 keys each), then the core tiles; the first
half (rows P_lo .. mid-1) walks tile st at raw step st, the second half tile
st + off_b; after n_rt - off_b raw steps both walk the core tiles, tile
st + off_b at step st.  Tile q sits in K slot q mod 5 and V slot q mod 4.
Each step issues V(st + off_b), which lands within the step, and K(st + off_b
+ 2), which lands within the next one; the prologue loads K(0 .. off_b) and
V(0 .. off_b - 1), and K(off_b + 1) lands in the first step.  A step reads
K of its tile and V of the tile before it (the deferred P.V); the flushes
read V of each half's last raw tile and of the last tile.

Checked over the workloads' item shapes and random ones: every tile a half's
rows see is on its walk, and every read finds its own tile in the slot, landed
and not replaced by a later load issued before the read.
"""
from __future__ import annotations

import random

BK = 64
OFF, NSK, NSV = 2, 5, 4


def n_core(t, g, w):
    return max(0, (t - w + 1) // g)


def win_lo(t, w):
    return max(0, t - w + 1)


def schedule(P_lo, Le, RP, g, w):
    P_hi = min(Le - 1, P_lo + RP - 1)
    n_ct = (n_core(P_hi, g, w) + BK - 1) // BK
    r0 = win_lo(P_lo, w) & ~(BK - 1)
    n_rt = (P_hi - r0) // BK + 1
    mid = P_lo + RP // 2
    a_last = (min(mid - 1, Le - 1) - r0) // BK
    b_first = (win_lo(min(mid, Le - 1), w) - r0) // BK
    off_b = max(0, min(OFF, b_first, n_rt - 1 - a_last))
    return dict(P_hi=P_hi, n_ct=n_ct, r0=r0, n_rt=n_rt, mid=mid, off_b=off_b,
                n_raw=n_rt - off_b, steps=n_rt - off_b + n_ct, n_tiles=n_rt + n_ct)


def tile(s, half, st):
    lead = s["off_b"] if half == 1 else 0
    return st + lead if st < s["n_raw"] else st + s["off_b"]


def tiles_seen(s, rows, Le, g, w):
    seen = set()
    for t in rows:
        if t >= Le:
            continue
        seen.update(range((win_lo(t, w) - s["r0"]) // BK, (t - s["r0"]) // BK + 1))
        seen.update(s["n_rt"] + c for c in range((n_core(t, g, w) + BK - 1) // BK))
    return seen


def loads(s):
    """(kind, tile, slot, issued at step, readable from step); prologue = step -1."""
    ob = s["off_b"]
    out = [("K", x, x % NSK, -1, 0) for x in range(ob + 1)]
    out += [("V", x, x % NSV, -1, 0) for x in range(ob)]
    out.append(("K", ob + 1, (ob + 1) % NSK, -1, 1))
    for st in range(s["steps"]):
        q = st + ob
        out.append(("V", q, q % NSV, st, st + 1))
        out.append(("K", q + 2, (q + 2) % NSK, st, st + 2))
    return out


def by_slot(ld):
    """Loads per (kind, slot), in issue order."""
    out = {}
    for x in ld:
        out.setdefault((x[0], x[2]), []).append(x)
    return out


def check_read(slots, kind, q, st, nslots):
    """A read of tile q at step st, after that step's own loads were issued."""
    slot = q % nslots
    into = [x for x in slots.get((kind, slot), ()) if x[3] <= st]
    assert into, (kind, q, st)
    last = into[-1]
    assert last[1] == q, f"{kind}({q}) at step {st}: slot {slot} holds tile {last[1]}"
    assert last[4] <= st, f"{kind}({q}) read at step {st} before it lands"


def check_item(P_lo, Le, g, w, RP=256):
    s = schedule(P_lo, Le, RP, g, w)
    halves = (range(P_lo, min(s["mid"], s["P_hi"] + 1)), range(s["mid"], s["P_hi"] + 1))
    for half, rows in enumerate(halves):
        walk = {tile(s, half, st) for st in range(s["steps"])}
        missing = tiles_seen(s, rows, Le, g, w) - walk
        assert not missing, (P_lo, Le, g, w, half, sorted(missing)[:4])
        assert all(0 <= q < s["n_tiles"] for q in walk)
    ld = loads(s)
    slots = by_slot(ld)
    for st in range(s["steps"]):
        for half in (0, 1):
            q = tile(s, half, st)
            check_read(slots, "K", q, st, NSK)
            if st not in (0, s["n_raw"]):  # a walk's first step multiplies P = 0
                check_read(slots, "V", q - 1, st, NSV)
    before = by_slot([x for x in ld if x[3] < s["n_raw"]])
    for half in (0, 1):  # the raw walk's flush, before step n_raw issues its loads
        check_read(before, "V", tile(s, half, s["n_raw"] - 1), s["n_raw"], NSV)
    check_read(slots, "V", s["n_tiles"] - 1, s["steps"], NSV)  # the last flush
    return s["off_b"]


def test_workload_shapes_every_item():
    """The MHA workloads (g 16, w 1024) at 32K and 128K, and the ragged
    lengths of the parity cases: every item."""
    for Le in (32768, 131072, 3500, 6000, 10240):
        for pb in range((Le + 255) // 256):
            check_item(pb * 256, Le, 16, 1024)


def test_halves_walk_apart_in_the_window_interior():
    """Away from the sequence start the leading half is two tiles ahead, so
    the raw walk takes 18 steps instead of the union's 20."""
    s = schedule(8192, 32768, 256, 16, 1024)
    assert s["off_b"] == 2 and s["n_rt"] == 20 and s["n_raw"] == 18


def test_random_shapes():
    rng = random.Random(5)
    offs = set()
    for _ in range(3000):
        w = rng.choice([1, 2, 5, 16, 63, 64, 65, 100, 500, 1023, 1024, 1025, 4096])
        g = rng.choice([1, 2, 3, 16, 100])
        Le = rng.randint(1, 40000)
        pb = rng.randrange((Le + 255) // 256)
        offs.add(check_item(pb * 256, Le, g, w))
    assert offs == {0, 1, 2}


def test_model_catches_a_short_ring():
    """The checks have teeth: with four K slots the leading half's prefetch
    replaces a tile the first half still reads."""
    global NSK
    saved, NSK = NSK, 4
    try:
        try:
            check_item(8192, 32768, 16, 1024)
        except AssertionError:
            return
        raise AssertionError("a four-slot K ring passed")
    finally:
        NSK = saved
