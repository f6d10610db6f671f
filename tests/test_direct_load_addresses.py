"""CPU model of the MFMA kernels' direct (global-to-LDS) loads: for every
tile, every 16-byte unit and every K step that the aligned and edge instances
load without bounds checks, the address the kernel forms must lie inside the
stored operand.  The model follows the kernel's own address arithmetic --
the row/column clamps of the edge instances, the 32-bit per-lane byte offsets
added to a wave-uniform base (which wrap if negative), and the K-row limit
that applies when a 16-byte piece can straddle the edge -- so a mistake there
shows up here, on the CPU, instead of as a memory fault on the GPU.

It needs the built library only for the kernel table (tile sizes per
instance); it launches nothing."""
import itertools

import numpy as np
import pytest

import fp32_gemm_major_amd as sg

KERNELS = sg.kernel_table() if __import__("os").path.exists(sg.LIBRARY) else []
MFMA_DIRECT = [k for k in KERNELS if k["variant"] == sg.SGEMM_VARIANT_MFMA
               and k["mode"] in (sg.SGEMM_MODE_ALIGNED, sg.SGEMM_MODE_EDGE)]


def ktiles_direct(mode, M, N, K, bk, ta, tb):
    """K steps the direct loads cover (the kernel's `ktiles`)."""
    straddle = mode == sg.SGEMM_MODE_EDGE and ((ta and M % 4) or (not tb and N % 4))
    if straddle:
        return (K - 1) // bk if K > 0 else 0
    return K // bk


def clamp(kcontig, o, origin, extent, old_rule=False):
    """Relative outer index of a unit whose outer index origin+o is past the
    edge (edge instances only)."""
    if kcontig:
        return extent - 1 - origin
    if old_rule:
        return extent - 4 - origin
    return extent - 4 - origin if extent - 4 > origin else 0


def operand_reads(kcontig, outer_tile, bk, extent, ld, steps, edge, old_rule=False):
    """Element ranges [first, first+4) of every direct load of one operand,
    relative to the operand's base pointer, over all tiles and K steps.

    kcontig: units are 4 consecutive k of one outer row (A as stored, B^T);
    else 4 consecutive outer indices of one k row (B as stored, A^T)."""
    tiles = -(-extent // outer_tile)
    firsts = []
    for t in range(tiles):
        origin = t * outer_tile
        if kcontig:
            o, k = np.meshgrid(np.arange(outer_tile), np.arange(0, bk, 4), indexing="ij")
        else:
            k, o = np.meshgrid(np.arange(bk), np.arange(0, outer_tile, 4), indexing="ij")
        o = o.ravel().astype(np.int64)
        k = k.ravel().astype(np.int64)
        if edge:
            past = origin + o >= extent
            if past.any():
                o = o.copy()
                o[past] = clamp(kcontig, None, origin, extent, old_rule)
        # lane byte offset as the kernel forms it: 32-bit unsigned
        rel = o * ld + k if kcontig else k * ld + o
        voff = (4 * rel) % (1 << 32)
        base = origin * ld if kcontig else origin  # tile origin, in elements
        for kt in range(steps):
            step = kt * bk if kcontig else kt * bk * ld
            firsts.append(base + step + voff // 4)
    return np.concatenate(firsts) if firsts else np.zeros(0, np.int64)


def check(k, M, N, K, lda, ldb, old_rule=False):
    ta, tb, bk = bool(k["transa"]), bool(k["transb"]), k["bk"]
    edge = k["mode"] == sg.SGEMM_MODE_EDGE
    steps = ktiles_direct(k["mode"], M, N, K, bk, ta, tb)
    bad = []
    # A: stored M x K (K-contiguous) or K x M (A^T)
    rows, cols = (K, M) if ta else (M, K)
    size = (rows - 1) * lda + cols
    f = operand_reads(not ta, k["bm"], bk, M, lda, steps, edge, old_rule)
    if f.size and (f.min() < 0 or f.max() + 4 > size):
        bad.append(("A", int(f.min()), int(f.max() + 4), size))
    # B: stored K x N (outer-contiguous) or N x K (B^T)
    rows, cols = (N, K) if tb else (K, N)
    size = (rows - 1) * ldb + cols
    f = operand_reads(tb, k["bn"], bk, N, ldb, steps, edge, old_rule)
    if f.size and (f.min() < 0 or f.max() + 4 > size):
        bad.append(("B", int(f.min()), int(f.max() + 4), size))
    return bad


def fits(k, M, N, K):
    """The host's rules for these instances (offsets are tiny here)."""
    ta, tb = k["transa"], k["transb"]
    if k["mode"] == sg.SGEMM_MODE_ALIGNED:
        return M % k["bm"] == 0 and N % k["bn"] == 0 and K % k["bk"] == 0
    return (not ta or M >= 4) and (tb or N >= 4)


SIZES = [1, 3, 4, 5, 6, 7, 63, 64, 65, 66, 67, 130, 257]
KS = [1, 3, 15, 16, 17, 31, 32, 33, 63, 64, 65, 96, 129]


@pytest.mark.parametrize("k", [k for k in MFMA_DIRECT if k["mode"] == sg.SGEMM_MODE_EDGE],
                         ids=lambda k: k["name"])
def test_edge_instances_stay_inside_the_operands(k):
    rng = np.random.default_rng(k["id"])
    combos = list(itertools.product(SIZES, SIZES, KS))
    picked = [combos[i] for i in rng.choice(len(combos), 160, replace=False)]
    picked += [(k["bm"] + 1, k["bn"] + 1, k["bk"]), (k["bm"] - 1, k["bn"] - 1, k["bk"] + 1),
               (2 * k["bm"] + 3, 2 * k["bn"] + 2, 2 * k["bk"])]
    for M, N, K in picked:
        if not fits(k, M, N, K):
            continue
        for pad in (0, 1):
            lda = (M if k["transa"] else K) + pad
            ldb = (K if k["transb"] else N) + pad
            assert check(k, M, N, K, lda, ldb) == [], (k["name"], M, N, K, pad)


@pytest.mark.parametrize("k", [k for k in MFMA_DIRECT if k["mode"] == sg.SGEMM_MODE_ALIGNED],
                         ids=lambda k: k["name"])
def test_aligned_instances_stay_inside_the_operands(k):
    for mt, nt, kt in [(1, 1, 1), (2, 3, 2), (3, 1, 4)]:
        M, N, K = mt * k["bm"], nt * k["bn"], kt * k["bk"]
        for pad in (0, 1, 3):
            lda = (M if k["transa"] else K) + pad
            ldb = (K if k["transb"] else N) + pad
            assert check(k, M, N, K, lda, ldb) == [], (k["name"], M, N, K, pad)


def test_the_model_catches_a_clamp_left_of_the_tile():
    """With the column clamp that ignores the tile origin, a 65-column B
    (last tile at column 64, clamp target 61) gives a negative lane offset
    that wraps to about 4 GiB: the model must flag it."""
    k = next(k for k in MFMA_DIRECT if k["mode"] == sg.SGEMM_MODE_EDGE
             and not k["transa"] and not k["transb"] and k["bn"] == 64)
    M, N, K = 64, 65, 2 * k["bk"]
    assert check(k, M, N, K, K, N) == []
    bad = check(k, M, N, K, K, N, old_rule=True)
    assert bad and bad[0][0] == "B" and bad[0][2] > 1 << 30
