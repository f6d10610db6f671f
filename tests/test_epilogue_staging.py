"""CPU model of the epilogues that stage accumulators through LDS.

The MFMA register layout holds, in register 4q + e of lane (li, lh), row li
and column 8q + 4lh + e of a 32x32 block.  The epilogues write those values
to LDS and read them back row by row so that every global C access of a wave
covers whole rows.  Checked, for the index arithmetic of the kernels:

* the FP32 tile kernel (store_tile_lds, mfma_sgemm.hpp): one 32x32 block per
  wave, rows of 32 floats, 16-byte unit u of row r stored at u ^ (r/2 % 8);
* the 16- and 8-bit kernels (lp_store_tile_lds, lowp_gemm.hpp): one 32-row
  block row of a WN-wide wave tile, rows padded to WN + 4 floats;

that every value read back is the one written for that (row, column), and
that each group of 16 lanes of an LDS write or read touches 16 distinct
16-byte bank groups (no bank conflicts).
"""
import pytest


def fp32_unit(r, u):
    return u ^ ((r >> 1) & 7)


def test_fp32_staging_round_trip_and_banks():
    store = {}
    for q in range(4):
        groups = {}
        for lane in range(64):
            li, lh = lane & 31, lane >> 5
            off = li * 32 + 4 * fp32_unit(li, 2 * q + lh)      # floats
            groups.setdefault(lane // 16, []).append((off // 4) % 16)
            for e in range(4):
                assert off + e not in store
                store[off + e] = (li, 8 * q + 4 * lh + e)
        assert all(len(set(g)) == 16 for g in groups.values()), q
    assert len(store) == 32 * 32
    for t in range(4):
        groups = {}
        for lane in range(64):
            r, cc = 8 * t + (lane >> 3), 4 * (lane & 7)
            off = r * 32 + 4 * fp32_unit(r, cc >> 2)
            groups.setdefault(lane // 16, []).append((off // 4) % 16)
            for e in range(4):
                assert store[off + e] == (r, cc + e)
        assert all(len(set(g)) == 16 for g in groups.values()), t


def test_fp32_staging_without_the_swizzle_conflicts():
    """Rows of 32 floats with no swizzle put the 16 rows of one register
    layout write on two bank groups (the model sees the conflict)."""
    groups = [((lane & 31) * 32 + 4 * (0 + (lane >> 5))) // 4 % 16 for lane in range(16)]
    assert len(set(groups)) == 2


@pytest.mark.parametrize("WN", [64, 128])
def test_lowp_staging_round_trip_and_banks(WN):
    LD, LPR = WN + 4, WN // 4
    RPI, NI = 64 // LPR, 32 // (64 // LPR)
    store = {}
    for j in range(WN // 32):
        for q in range(4):
            groups = {}
            for lane in range(64):
                li, lh = lane & 31, lane >> 5
                off = li * LD + 32 * j + 8 * q + 4 * lh
                groups.setdefault(lane // 16, []).append((off // 4) % 16)
                for e in range(4):
                    assert off + e not in store
                    store[off + e] = (li, 32 * j + 8 * q + 4 * lh + e)
            assert all(len(set(g)) == 16 for g in groups.values()), (j, q)
    assert len(store) == 32 * WN
    for t in range(NI):
        groups = {}
        for lane in range(64):
            rr, cc = lane // LPR, 4 * (lane % LPR)
            off = (t * RPI + rr) * LD + cc
            groups.setdefault(lane // 16, []).append((off // 4) % 16)
            for e in range(4):
                assert store[off + e] == (t * RPI + rr, cc + e)
        assert all(len(set(g)) == 16 for g in groups.values()), t
