"""CPU model of the epilogues that stage accumulators through LDS.

The MFMA register layout holds, in register 4q + e of lane (li, lh), row li
and column 8q + 4lh + e of a 32x32 block.  The epilogues write those values
to LDS and read them back row by row so that every global C access of a wave
covers whole rows.  Checked, for the index arithmetic of the kernels:

* the FP32 tile kernel (store_tile_lds, mfma_sgemm.hpp): one 32x32 block per
  wave, rows of 32 floats, 16-byte unit u of row r stored at u ^ (r % 8);
* the 16- and 8-bit kernels (lp_store_tile_lds, lowp_gemm.hpp): one 32-row
  block row of a WN-wide wave tile, rows padded to WN + 4 floats;

that every value read back is the one written for that (row, column), and
that no LDS access has a bank conflict under the rule gfx950 follows for
16-byte accesses, as measured with SQ_LDS_BANK_CONFLICT on one-wave kernels
repeating fixed address patterns:

* a 16-byte write is served 8 lanes at a time over 32 four-byte banks: the
  8 lanes' 16-byte units must differ modulo 8;
* a 16-byte read is served 16 lanes at a time over 64 banks: the 16 lanes'
  units must differ modulo 16.

(On those kernels, 8 lanes writing units 0-7 and 8 more writing units 16-23
counted no conflict while the same pattern read counted one per pass; 8
lanes writing units with only four distinct values modulo 8 but eight modulo
16 counted a two-way conflict.)
"""
import pytest


def write_conflict_free(units):
    """Units (16-byte, per lane, 64 lanes) of one 16-byte write."""
    return all(len({u % 8 for u in units[g:g + 8]}) == 8 for g in range(0, 64, 8))


def read_conflict_free(units):
    """Units (16-byte, per lane, 64 lanes) of one 16-byte read."""
    return all(len({u % 16 for u in units[g:g + 16]}) == 16 for g in range(0, 64, 16))


def fp32_unit(r, u):
    return u ^ (r & 7)


def test_bank_rule_matches_the_measured_patterns():
    """The patterns the rule was measured on, with the outcome the counter
    gave: a guard against editing the rule into something the hardware did
    not show."""
    lanes = range(64)
    contiguous = [l for l in lanes]
    eight_apart = [(l & 7) + 16 * (l >> 3) for l in lanes]
    half_row_swizzle = [(l & 31) * 8 + ((l >> 5) ^ (((l & 31) >> 1) & 7)) for l in lanes]
    padded_rows = [(l >> 3) * 9 + (l & 7) for l in lanes]
    assert write_conflict_free(contiguous) and read_conflict_free(contiguous)
    assert write_conflict_free(eight_apart) and not read_conflict_free(eight_apart)
    assert not write_conflict_free(half_row_swizzle) and read_conflict_free(half_row_swizzle)
    assert write_conflict_free(padded_rows) and not read_conflict_free(padded_rows)


def test_fp32_staging_round_trip_and_banks():
    store = {}
    for q in range(4):
        units = []
        for lane in range(64):
            li, lh = lane & 31, lane >> 5
            off = li * 32 + 4 * fp32_unit(li, 2 * q + lh)      # floats
            units.append(off // 4)
            for e in range(4):
                assert off + e not in store
                store[off + e] = (li, 8 * q + 4 * lh + e)
        assert write_conflict_free(units), q
    assert len(store) == 32 * 32
    for t in range(4):
        units = []
        for lane in range(64):
            r, cc = 8 * t + (lane >> 3), 4 * (lane & 7)
            off = r * 32 + 4 * fp32_unit(r, cc >> 2)
            units.append(off // 4)
            for e in range(4):
                assert store[off + e] == (r, cc + e)
        assert read_conflict_free(units), t


def test_fp32_kernel_constants_match_the_swizzle():
    """The kernel folds the swizzle into per-lane constants: writes at unit
    2q ^ xw with xw = lh ^ (li % 8), reads at unit xr = (cc/4) ^ rr of row
    8t + rr."""
    for lane in range(64):
        li, lh = lane & 31, lane >> 5
        xw = lh ^ (li & 7)
        for q in range(4):
            assert (2 * q) ^ xw == fp32_unit(li, 2 * q + lh)
        rr, cc = lane >> 3, 4 * (lane & 7)
        xr = (cc >> 2) ^ rr
        for t in range(4):
            assert xr == fp32_unit(8 * t + rr, cc >> 2)


def test_fp32_staging_half_row_swizzle_conflicts_on_writes():
    """u ^ (r/2 % 8) spreads 16 consecutive rows over 16 bank groups, but the
    8 rows one write serves at a time fall on four units: two-way
    conflicts, which the counter showed for that layout."""
    for q in range(4):
        units = [(l & 31) * 8 + ((2 * q + (l >> 5)) ^ (((l & 31) >> 1) & 7)) for l in range(64)]
        assert not write_conflict_free(units)


def test_fp32_staging_without_the_swizzle_conflicts():
    """Rows of 32 floats with no swizzle put the 8 rows of one register
    layout write on one unit."""
    units = [(l & 31) * 8 + (l >> 5) for l in range(64)]
    assert not write_conflict_free(units)
    assert len({u % 8 for u in units[:8]}) == 1


@pytest.mark.parametrize("WN", [64, 128])
def test_lowp_staging_round_trip_and_banks(WN):
    LD, LPR = WN + 4, WN // 4
    RPI, NI = 64 // LPR, 32 // (64 // LPR)
    store = {}
    for j in range(WN // 32):
        for q in range(4):
            units = []
            for lane in range(64):
                li, lh = lane & 31, lane >> 5
                off = li * LD + 32 * j + 8 * q + 4 * lh
                units.append(off // 4)
                for e in range(4):
                    assert off + e not in store
                    store[off + e] = (li, 32 * j + 8 * q + 4 * lh + e)
            assert write_conflict_free(units), (j, q)
    assert len(store) == 32 * WN
    for t in range(NI):
        units = []
        for lane in range(64):
            rr, cc = lane // LPR, 4 * (lane % LPR)
            off = (t * RPI + rr) * LD + cc
            units.append(off // 4)
            for e in range(4):
                assert store[off + e] == (t * RPI + rr, cc + e)
        assert read_conflict_free(units), t
