"""CPU model of the stream-K kernels' work split (no GPU): the tiles x K-steps
iteration space cut into G equal contiguous ranges, the partial-tile slots
each workgroup writes, and the fixup assignment.  The model follows the
kernels' integer formulas -- range bounds b(h) = floor(h*W/G), slot 2h for a
workgroup's first part and 2h+1 for its last, the fixup done by a split
tile's last owner, owner(i) = floor(((i+1)*G - 1) / W) -- and checks that
every (tile, K step) is accumulated exactly once, every tile is stored
exactly once, and every fixup reads exactly the partials of its tile in K
order."""
import random

import pytest


def bound(W, G, h):
    return W * h // G


def sk_parts(tiles, steps, G):
    """What the stream-K kernel does: per workgroup, the parts it runs and
    where each goes ('C' or a slot index)."""
    W = tiles * steps
    out = []
    for h in range(G):
        b0, b1 = bound(W, G, h), bound(W, G, h + 1)
        i = b0
        while i < b1:
            t = i // steps
            ts = t * steps
            s0 = i - ts
            s1 = min(steps, b1 - ts)
            if s0 == 0 and s1 == steps:
                dest = "C"
            else:
                dest = 2 * h + (0 if i == b0 else 1)
            out.append((h, t, s0, s1, dest))
            i = ts + s1
    return out


def fixups(tiles, steps, G):
    """What the fixup kernel does: per workgroup that fixes a tile, the tile
    and the slots it adds, in order."""
    W = tiles * steps
    out = []
    for h in range(G):
        b0, b1 = bound(W, G, h), bound(W, G, h + 1)
        if b0 >= b1:
            continue
        t = b0 // steps
        ts = t * steps
        if b0 == ts or b1 < ts + steps:
            continue
        first = ((ts + 1) * G - 1) // W
        slots = []
        for o in range(first, h + 1):
            bo = bound(W, G, o)
            if bo >= bound(W, G, o + 1):
                continue
            slots.append(2 * o + (0 if bo >= ts else 1))
        out.append((h, t, slots))
    return out


def check(tiles, steps, G):
    parts = sk_parts(tiles, steps, G)
    fix = fixups(tiles, steps, G)
    covered = {}
    for h, t, s0, s1, dest in parts:
        assert 0 <= s0 < s1 <= steps
        for s in range(s0, s1):
            assert (t, s) not in covered, ("step twice", t, s)
            covered[(t, s)] = (h, dest)
    assert len(covered) == tiles * steps
    slots_written = [dest for *_, dest in parts if dest != "C"]
    assert len(slots_written) == len(set(slots_written))
    assert all(0 <= d < 2 * G for d in slots_written)
    stored = {}
    for h, t, s0, s1, dest in parts:
        if dest == "C":
            assert t not in stored
            stored[t] = "direct"
    fixed_tiles = [t for _, t, _ in fix]
    assert len(fixed_tiles) == len(set(fixed_tiles))
    for h, t, slots in fix:
        assert t not in stored, ("tile both stored and fixed", t)
        stored[t] = "fixup"
        # exactly the partials of tile t, in K order
        want = [dest for _, tt, s0, _, dest in sorted(
            (p for p in parts if p[1] == t), key=lambda p: p[2])]
        assert "C" not in want and slots == want, (t, slots, want)
    assert sorted(stored) == list(range(tiles))
    # every partial slot is read by exactly one fixup
    read = [s for _, _, slots in fix for s in slots]
    assert sorted(read) == sorted(slots_written)


@pytest.mark.parametrize("tiles,steps,G", [
    (1, 1, 1), (1, 1, 4), (1, 7, 4), (3, 1, 8), (256, 129, 256), (289, 129, 256),
    (1089, 257, 512), (384, 13, 256), (384, 13, 512), (6, 4, 512), (2752, 256, 512),
    (5, 3, 7), (7, 5, 3), (100, 1, 256), (1, 1000, 256)])
def test_partition(tiles, steps, G):
    check(tiles, steps, G)


def test_partition_random():
    rng = random.Random(5)
    for _ in range(300):
        check(rng.randint(1, 60), rng.randint(1, 40), rng.randint(1, 70))


def test_owner_formula():
    """owner(i) = floor(((i+1)G - 1)/W) is the workgroup whose range holds i."""
    rng = random.Random(9)
    for _ in range(200):
        W, G = rng.randint(1, 500), rng.randint(1, 90)
        for i in range(W):
            h = ((i + 1) * G - 1) // W
            assert bound(W, G, h) <= i < bound(W, G, h + 1)


def test_workspace_slots_match_the_host_size():
    """Slots 2h and 2h+1 of a grid of G: 2G slots, the size the host asks for."""
    for G in (1, 256, 512):
        parts = sk_parts(1000, 37, G)
        assert max((d for *_, d in parts if d != "C"), default=-1) < 2 * G


def xcd_position(wg, G, xcds=8):
    return (wg % xcds) * (G // xcds) + wg // xcds if G % xcds == 0 else wg


@pytest.mark.parametrize("G", [1, 7, 8, 16, 24, 256, 512, 1000, 1024])
def test_xcd_positions_are_a_permutation(G):
    """Workgroup ids are renumbered to positions; every position must be
    owned exactly once, and one XCD's workgroups (ids congruent mod 8)
    must hold one contiguous run of positions when G is a multiple of 8."""
    pos = [xcd_position(w, G) for w in range(G)]
    assert sorted(pos) == list(range(G))
    if G % 8 == 0:
        for x in range(8):
            run = sorted(pos[w] for w in range(x, G, 8))
            assert run == list(range(run[0], run[0] + G // 8))
