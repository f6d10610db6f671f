"""CPU model of the 16- and 8-bit kernels' outer-contiguous LDS tiles.

An operand stored with its outer index (m or n) contiguous is copied into LDS
by direct loads, slot by slot, with its 16-byte units XOR-swizzled per row of
k, and its MFMA fragments are gathered by transposing LDS reads.  The model
follows the kernel's index arithmetic (lowp_gemm.hpp: the slot mapping of the
direct loads, lp_oc_swz and read_tr) and the transposing read's lane mapping
as measured on the device with an in-bounds probe: within each group of 16
lanes, lane i receives, as element e, element i % 4 of the four 16-bit values
that lane 4e + i // 4 points at.  It checks that every lane of a 32x32x16
fragment gets k = 16q + 8*(lane // 32) + t (t = 0..7) of outer index
lane % 32, as a K-contiguous fragment would, and that the reads are free of
bank conflicts.

8-bit tiles (every mode) use ds_read_b64_tr_b8, whose lane mapping, measured
the same way, is: within each group of 16 lanes, lane i receives, as byte e,
byte i % 8 of the eight that lane 2e + i // 8 points at.  The model follows
lp_oc_swz8 and read_tr8 and checks that every lane of a 32x32x64 fragment
gets k = 64q + 32*(lane // 32) + t (t = 0..31) of outer index lane % 32.
"""
import pytest


def oc_swz(X, k):
    return 4 * (k & 3) if X >= 128 else 4 * ((k >> 1) & 1)


def fill_tile(X):
    """LDS byte offset -> (k, outer) of the element stored there, after the
    direct loads of one K step (64 k) of a tile X wide."""
    units_per_row = X // 8
    lds = {}
    for u in range(64 * units_per_row):           # slot u: 16 bytes at 16u
        k, p = divmod(u, units_per_row)
        c = p ^ oc_swz(X, k)                       # logical unit loaded there
        assert 0 <= c < units_per_row
        for t in range(8):
            lds[16 * u + 2 * t] = (k, 8 * c + t)
    assert len(lds) == 64 * X                      # every element exactly once
    return lds


def tr_read(lds, addr_of_lane):
    """The transposing read: per lane, four 16-bit values."""
    out = {}
    for lane in range(64):
        g, i = divmod(lane, 16)
        vals = []
        for e in range(4):
            src = 16 * g + 4 * e + i // 4
            vals.append(lds[addr_of_lane(src) + 2 * (i % 4)])
        out[lane] = vals
    return out


def read_tr_offsets(X, o_block, q):
    """Byte offset each lane passes to the first of its two reads."""
    def off(lane):
        lh = lane >> 5
        e, r = (lane & 15) >> 2, lane & 3
        k = 16 * q + 8 * lh + e
        o = o_block + 16 * ((lane >> 4) & 1) + 4 * r
        return k * 2 * X + 16 * ((o >> 3) ^ oc_swz(X, k)) + 2 * (o & 7)
    return off


@pytest.mark.parametrize("X", [64, 128, 256])
def test_transposed_fragments_match_k_contiguous_order(X):
    lds = fill_tile(X)
    for o_block in range(0, X, 32):
        for q in range(4):
            off = read_tr_offsets(X, o_block, q)
            lo = tr_read(lds, off)
            hi = tr_read(lds, lambda lane: off(lane) + 4 * 2 * X)
            for lane in range(64):
                got = lo[lane] + hi[lane]
                want = [(16 * q + 8 * (lane // 32) + t, o_block + lane % 32)
                        for t in range(8)]
                assert got == want, (X, o_block, q, lane)


@pytest.mark.parametrize("X", [64, 128, 256])
def test_transposed_reads_have_no_bank_conflicts(X):
    """Each half-wave (32 lanes x 8 bytes = 256 bytes) of a transposing read
    touches every 16-byte bank group of a 256-byte LDS line exactly twice (two
    8-byte halves of one unit)."""
    for o_block in range(0, X, 32):
        for q in range(4):
            off = read_tr_offsets(X, o_block, q)
            for half in (0, 1):
                groups = {}
                for lane in range(32 * half, 32 * half + 32):
                    b = off(lane)
                    groups.setdefault((b // 16) % 16, set()).add(b % 16)
                assert len(groups) == 16, (X, o_block, q, half)
                assert all(v == {0, 8} for v in groups.values())


@pytest.mark.parametrize("X", [64, 128, 256])
def test_direct_load_slots_stay_coalesced(X):
    """The 64 lanes of one direct load read whole 128-byte pieces of global
    rows: the swizzle only permutes units inside 64- or 256-byte groups."""
    units_per_row = X // 8
    for first in range(0, 64 * units_per_row, 64):
        rows = {}
        for u in range(first, first + 64):
            k, p = divmod(u, units_per_row)
            rows.setdefault(k, set()).add(p ^ oc_swz(X, k))
        for k, units in rows.items():
            assert units == set(range(min(units), min(units) + len(units)))
            assert len(units) % 8 == 0


# ---- 8-bit tiles ---------------------------------------------------------------

def oc_swz8(X, k):
    return 2 * {256: k & 7, 128: (k >> 1) & 3, 64: (k >> 2) & 1}[X]


def fill_tile8(X):
    """LDS byte offset -> (k, outer) after one K step (128 k) of an 8-bit tile
    X wide (the direct loads' and the register-staged loads' slot mapping)."""
    units_per_row = X // 16
    lds = {}
    for u in range(128 * units_per_row):
        k, p = divmod(u, units_per_row)
        c = p ^ oc_swz8(X, k)
        assert 0 <= c < units_per_row
        for t in range(16):
            lds[16 * u + t] = (k, 16 * c + t)
    assert len(lds) == 128 * X
    return lds


def tr8_read(lds, addr_of_lane):
    """The 8-bit transposing read: per lane, eight bytes."""
    out = {}
    for lane in range(64):
        g, i = divmod(lane, 16)
        out[lane] = [lds[addr_of_lane(16 * g + 2 * e + i // 8) + i % 8] for e in range(8)]
    return out


def read_tr8_offsets(X, o_block, q, j):
    """Byte offset each lane passes to read j (0..3) of a fragment."""
    def off(lane):
        lh = lane >> 5
        e = (lane & 15) >> 1
        o = o_block + 16 * ((lane >> 4) & 1) + 8 * (lane & 1)
        k = 64 * q + 32 * lh + 8 * j + e
        return k * X + 16 * ((o >> 4) ^ oc_swz8(X, k)) + (o & 15)
    return off


@pytest.mark.parametrize("X", [64, 128, 256])
def test_8bit_transposed_fragments_match_k_contiguous_order(X):
    lds = fill_tile8(X)
    for o_block in range(0, X, 32):
        for q in range(2):
            reads = [tr8_read(lds, read_tr8_offsets(X, o_block, q, j)) for j in range(4)]
            for lane in range(64):
                got = [v for j in range(4) for v in reads[j][lane]]
                want = [(64 * q + 32 * (lane // 32) + t, o_block + lane % 32) for t in range(32)]
                assert got == want, (X, o_block, q, lane)


@pytest.mark.parametrize("X", [64, 128, 256])
def test_8bit_transposed_reads_have_no_bank_conflicts(X):
    """Each half-wave of an 8-bit transposing read touches every 16-byte bank
    group of a 256-byte LDS line exactly twice (its two 8-byte halves)."""
    for o_block in range(0, X, 32):
        for q in range(2):
            for j in range(4):
                off = read_tr8_offsets(X, o_block, q, j)
                for half in (0, 1):
                    groups = {}
                    for lane in range(32 * half, 32 * half + 32):
                        b = off(lane)
                        assert b % 8 == 0
                        groups.setdefault((b // 16) % 16, set()).add(b % 16)
                    assert len(groups) == 16, (X, o_block, q, j, half)
                    assert all(v == {0, 8} for v in groups.values())


def test_8bit_swizzle_without_the_factor_two_conflicts():
    """The two lane groups of a half-wave read units c and c ^ 1: an XOR by
    k & 7 alone maps both onto the same eight bank groups (the model sees the
    two-way conflict)."""
    X, k0, c = 256, 0, 0
    groups = {}
    for e in range(8):
        for unit in (c, c ^ 1):
            groups.setdefault(((k0 + e) * X // 16 + (unit ^ ((k0 + e) & 7))) % 16, 0)
            groups[((k0 + e) * X // 16 + (unit ^ ((k0 + e) & 7))) % 16] += 1
    assert len(groups) == 8 and max(groups.values()) == 2


@pytest.mark.parametrize("X", [64, 128, 256])
def test_8bit_direct_load_slots_stay_coalesced(X):
    """The 64 lanes of one direct load read whole rows of k (X bytes each):
    the swizzle only permutes units inside a row."""
    units_per_row = X // 16
    for first in range(0, 128 * units_per_row, 64):
        rows = {}
        for u in range(first, first + 64):
            k, p = divmod(u, units_per_row)
            rows.setdefault(k, set()).add(p ^ oc_swz8(X, k))
        for k, units in rows.items():
            assert units == set(range(units_per_row)), (X, k)
