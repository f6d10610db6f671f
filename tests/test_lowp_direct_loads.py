"""CPU model of the 16- and 8-bit kernels' direct (global-to-LDS) loads: for every
tile, every 16-byte piece and every K step that the aligned and edge
instances load without bounds checks -- including the look-ahead steps past
the end of K, which the kernel clamps to the last direct-load step -- the
elements read (8 of a 16-bit format, 16 of an 8-bit one) must lie inside the
stored operand.  The model follows the
kernel's own arithmetic (lowp_gemm.hpp): the slot-to-piece mapping of each
layout, the row clamp (K-contiguous) and the piece clamp (outer-contiguous)
of the edge kernels, the 32-bit per-lane byte offsets added to a wave-uniform
base, and the rule that leaves the last K row out of the direct loads when a
piece can straddle the M or N edge.  It needs the built library only for the
kernel table; it launches nothing."""
import numpy as np
import pytest

import fp32_gemm_major_amd as sg

KERNELS = sg.lowp_kernel_table() if __import__("os").path.exists(sg.LIBRARY) else []
# (the one-pass small-M kernels make no direct loads: tests/test_lowp_gemv_model.py)
DIRECT = [k for k in KERNELS if k["mode"] in (sg.SGEMM_MODE_ALIGNED, sg.SGEMM_MODE_EDGE)
          and k["dtype"] in (sg.SGEMM_DTYPE_BF16, sg.SGEMM_DTYPE_FP8_E4M3)
          and "_G16x16_" not in k["name"]]


def elem_bytes(dtype):
    return 1 if dtype >= sg.SGEMM_DTYPE_FP8_E4M3 else 2


def oc_swz(X, k, UE=8):
    """Unit swizzle of an outer-contiguous tile X elements wide (lp_oc_swz for
    16-bit elements, lp_oc_swz8 for 8-bit ones)."""
    if UE == 8:
        return 4 * (k & 3) if X >= 128 else 4 * ((k >> 1) & 1)
    return 2 * {256: k & 7, 128: (k >> 1) & 3, 64: (k >> 2) & 1}[X]


def direct_steps(edge, M, N, K, ta, tb, BK, UE=8):
    """K steps the direct loads cover (the kernel's kd)."""
    if not edge:
        return K // BK
    straddle = (ta and M % UE) or (not tb and N % UE)
    return (K - 1) // BK if straddle else K // BK


def piece_offsets(kcontig, X, extent, origin, ld, edge, BK, UE):
    """Element offset, relative to the tile's origin at K step 0, of the
    first of the UE elements of every slot of one operand tile."""
    units = X * BK // UE
    u = np.arange(units)
    if kcontig:                       # row r = u // 8, unit c = (u % 8) ^ ((r // 2) % 8)
        r = u // 8
        c = (u % 8) ^ ((r >> 1) & 7)
        if edge:
            r = np.where(origin + r >= extent, extent - 1 - origin, r)
        return r * ld + UE * c
    k = u // (X // UE)                # outer-contiguous: row k, unit swizzled by k
    c = (u % (X // UE)) ^ np.array([oc_swz(X, int(x), UE) for x in k])
    o = UE * c
    if edge:
        past = origin + o >= extent
        o = np.where(past, extent - UE - origin if extent - UE > origin else 0, o)
    return k * ld + o


def operand_reads(kcontig, X, extent, K, ld, steps, edge, BK=64, UE=8):
    """[first, last] element of every direct load of one operand, relative
    to its base, over all tiles and every step the kernel issues (0 .. kd-1,
    and the clamped look-ahead steps, which repeat step kd-1)."""
    lo, hi = [], []
    for origin in range(0, extent, X):
        off = piece_offsets(kcontig, X, extent, origin, ld, edge, BK, UE)
        # the per-lane byte offsets are 32-bit: negative ones would wrap
        assert off.min() >= 0 and (16 // UE) * off.max() < 2 ** 32
        base = origin * ld if kcontig else origin
        for kt in range(steps):       # look-ahead steps repeat steps-1: nothing new
            step = kt * BK if kcontig else kt * BK * ld
            first = base + step + off
            lo.append(first.min())
            hi.append((first + UE - 1).max())
    return (min(lo), max(hi)) if lo else (0, -1)


CASES = [(4096, 4096, 4096), (1000, 1500, 777), (150, 133, 192), (152, 136, 192),
         (150, 133, 40), (150, 133, 129), (64, 64, 64), (8, 9, 65), (300, 8, 128),
         (257, 255, 1000), (16, 300, 256), (300, 16, 384), (136, 264, 256)]


@pytest.mark.parametrize("k", DIRECT, ids=[k["name"] for k in DIRECT])
def test_direct_loads_stay_inside_the_operands(k):
    edge = k["mode"] == sg.SGEMM_MODE_EDGE
    ta, tb = bool(k["transa"]), bool(k["transb"])
    BK, UE = k["bk"], 16 // elem_bytes(k["dtype"])
    assert BK * elem_bytes(k["dtype"]) == 128
    for (M, N, K) in CASES:
        if not edge and (M % k["bm"] or N % k["bn"] or K % BK):
            continue
        if edge and ((ta and M < UE) or (not tb and N < UE)):
            continue
        for pad in (0, 1, 7):
            lda = (M if ta else K) + pad
            ldb = (K if tb else N) + pad
            kd = direct_steps(edge, M, N, K, ta, tb, BK, UE)
            a_rows, a_cols = (K, M) if ta else (M, K)
            b_rows, b_cols = (N, K) if tb else (K, N)
            a_lo, a_hi = operand_reads(not ta, k["bm"], M, K, lda, kd, edge, BK, UE)
            b_lo, b_hi = operand_reads(tb, k["bn"], N, K, ldb, kd, edge, BK, UE)
            tag = f"{k['name']} {M}x{N}x{K} pad {pad}"
            assert a_lo >= 0 and a_hi <= (a_rows - 1) * lda + a_cols - 1, tag + " A"
            assert b_lo >= 0 and b_hi <= (b_rows - 1) * ldb + b_cols - 1, tag + " B"


def test_straddle_rule_is_needed():
    """Without leaving the last K row out, a straddling piece of the last row
    would read past the end of B (the model catches it)."""
    M, N, K = 150, 133, 192
    ldb = N
    with pytest.raises(AssertionError):
        lo, hi = operand_reads(False, 64, N, K, ldb, K // 64, True)
        assert hi <= (K - 1) * ldb + N - 1


def test_straddle_rule_is_needed_for_8bit_pieces():
    """An 8-bit piece is 16 elements: N = 136 is a multiple of 8 but not of
    16, so the rule must leave the last K row out there too (the model
    catches the read past the end of B without it)."""
    M, N, K = 150, 136, 256
    ldb = N
    assert direct_steps(True, M, N, K, False, False, 128, 16) == (K - 1) // 128
    with pytest.raises(AssertionError):
        lo, hi = operand_reads(False, 128, N, K, ldb, K // 128, True, 128, 16)
        assert hi <= (K - 1) * ldb + N - 1
