"""CPU model of the stream-K kernels' work split (no GPU): the whole tiles
taken one per workgroup first (D of them, from the rule of sk_dp_tiles), the
other tiles' K-steps iteration space cut into G equal contiguous ranges, the
partial-tile slots each workgroup writes, and the fixup assignment.  The
model follows the kernels' integer formulas -- whole tiles h, h+G, ... < D,
range bounds b(h) = floor(h*W/G) with W = (tiles-D)*steps, slot 2h for a
workgroup's first part and 2h+1 for its last, the fixup done by a split
tile's last owner, owner(i) = floor(((i+1)*G - 1) / W) -- and checks that
every (tile, K step) is accumulated exactly once, every tile is stored
exactly once, and every fixup reads exactly the partials of its tile in K
order."""
import random

import pytest


def bound(W, G, h):
    return W * h // G


def dp_tiles(tiles, G, steps):
    full, rem = divmod(tiles, G)
    if full == 0:
        return 0
    if rem == 0:
        return tiles
    if rem * steps >= G * max(steps // 4, 2):
        return full * G
    return (full - 1) * G


def sk_parts(tiles, steps, G, dp=0):
    """What the stream-K kernel does: per workgroup, the parts it runs and
    where each goes ('C' or a slot index)."""
    W = (tiles - dp) * steps
    out = []
    for h in range(G):
        for t in range(h, dp, G):
            out.append((h, t, 0, steps, "C"))
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
            out.append((h, dp + t, s0, s1, dest))
            i = ts + s1
    return out


def fixups(tiles, steps, G, dp=0):
    """What the fixup kernel does: per split tile, the slots it adds, in
    order (owners from owner(u*steps) to owner((u+1)*steps - 1); a tile
    with one owner is not fixed)."""
    W = (tiles - dp) * steps
    out = []
    for u in range(tiles - dp):
        ts = u * steps
        first = ((ts + 1) * G - 1) // W
        last = ((ts + steps) * G - 1) // W
        if first == last:
            continue
        slots = []
        for o in range(first, last + 1):
            bo = bound(W, G, o)
            if bo >= bound(W, G, o + 1):
                continue
            slots.append(2 * o + (0 if bo >= ts else 1))
        out.append((last, dp + u, slots))
    return out


def check(tiles, steps, G, dp=0):
    assert dp % G == 0 and 0 <= dp <= tiles
    parts = sk_parts(tiles, steps, G, dp)
    fix = fixups(tiles, steps, G, dp)
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
    check(tiles, steps, G, dp_tiles(tiles, G, steps))


def test_partition_random():
    rng = random.Random(5)
    for _ in range(300):
        tiles, steps, G = rng.randint(1, 60), rng.randint(1, 40), rng.randint(1, 70)
        check(tiles, steps, G)
        check(tiles, steps, G, dp_tiles(tiles, G, steps))
        check(tiles, steps, G, G * rng.randint(0, tiles // G))


def test_whole_tile_rule():
    """The last partial round alone is split when each workgroup's share is
    at least max(steps // 4, 2) K steps, else the round before it too; a
    grid with no whole round splits everything, an exact multiple nothing."""
    assert dp_tiles(384, 256, 13) == 256      # 128 tiles over 256: 6.5 steps each
    assert dp_tiles(264, 256, 13) == 0        # 8 tiles: 0.4 steps each
    assert dp_tiles(520, 256, 13) == 256      # 8 left: split the round before
    assert dp_tiles(200, 256, 64) == 0
    assert dp_tiles(512, 256, 64) == 512
    for tiles in range(1, 3000, 7):
        for G, steps in ((256, 13), (512, 64), (256, 1)):
            dp = dp_tiles(tiles, G, steps)
            assert dp % G == 0 and 0 <= dp <= tiles
            if 0 < dp < tiles and steps >= 2:
                assert (tiles - dp) * steps >= G * max(steps // 4, 2)


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
        for dp in (0, dp_tiles(1000, G, 37)):
            parts = sk_parts(1000, 37, G, dp)
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


# (BM, BN, WM, WN) of the MFMA tile shapes
SHAPES = [(256, 256, 128, 64), (256, 128, 64, 64), (128, 128, 64, 64), (64, 64, 32, 32)]


@pytest.mark.parametrize("bm,bn,wm_,wn_", SHAPES)
def test_fixup_piece_decode(bm, bn, wm_, wn_):
    """A partial slot holds lane l's four accumulators q of block (i, j) of
    wave wmn at float 4c, c = (((wmn*FM + i)*FN + j)*4 + q)*64 + l; the
    fixup decodes c back to a row and four columns of the tile.  The decode
    must invert the layout, and the pieces must cover the tile once."""
    FM, FN, WAVES_N = wm_ // 32, wn_ // 32, bn // wn_
    waves = (bm // wm_) * WAVES_N
    seen = set()
    for wmn in range(waves):
        wm, wn = divmod(wmn, WAVES_N)
        for i in range(FM):
            for j in range(FN):
                for q in range(4):
                    for lane in range(64):
                        li, lh = lane & 31, lane >> 5
                        row = wm * wm_ + li + 32 * i        # the accumulator's place
                        col = wn * wn_ + 4 * lh + 32 * j + 8 * q
                        c = (((wmn * FM + i) * FN + j) * 4 + q) * 64 + lane
                        # the fixup's decode
                        dl, dq = c & 63, (c >> 6) & 3
                        dj, di = (c >> 8) % FN, (c >> 8) // FN % FM
                        dw = (c >> 8) // (FN * FM)
                        drow = (dw // WAVES_N) * wm_ + di * 32 + (dl & 31)
                        dcol = (dw % WAVES_N) * wn_ + dj * 32 + (dl >> 5) * 4 + 8 * dq
                        assert (drow, dcol) == (row, col)
                        for e in range(4):
                            assert (row, col + e) not in seen
                            seen.add((row, col + e))
    assert len(seen) == bm * bn
