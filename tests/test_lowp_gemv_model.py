"""CPU model of the one-pass small-M kernels (lp_gemv_kernel, lowp_gemv.hpp).

The index arithmetic of the kernel, replayed per lane for a range of shapes,
leading dimensions and both storages of A: every byte it reads lies inside
the operand windows the C ABI validates; the lanes' pieces cover every k of
every row of B exactly once, each piece paired with the same k of the
matching row of A (what the MFMA needs of its two operands); every output
(m < M, n < N) is written exactly once and nothing else is written.
"""
import itertools

import pytest

import fp32_gemm_major_amd as sg

KERNELS = sg.lowp_kernel_table() if __import__("os").path.exists(sg.LIBRARY) else []
GEMV = [k for k in KERNELS if "_G16x16_" in k["name"]]

WAVES, COLS = 8, 16


def fmt(dtype):
    """(element bytes, elements per 16-byte piece, k per block, pieces per lane)"""
    if dtype >= sg.SGEMM_DTYPE_FP8_E4M3:
        return 1, 16, 128, 2
    return 2, 8, 32, 1


def piece_k(dtype, q, p):
    return 16 * q + 64 * p if dtype >= sg.SGEMM_DTYPE_FP8_E4M3 else 8 * q


def replay(dtype, ta, M, N, K, lda, ldb, ldc):
    esz, ue, kb, pc = fmt(dtype)
    batch = 8 // pc
    a_end = ((K - 1) * lda + M) if ta else ((M - 1) * lda + K)  # elements
    b_end = (N - 1) * ldb + K
    used = {}      # (n, k) -> number of times the pair (B[n,k], A[m,k]) is multiplied
    written = {}
    nblk = -(-K // kb)
    per = -(-nblk // WAVES)
    for wg in range(-(-N // COLS)):
        for wave in range(WAVES):
            b0, b1 = wave * per, min(wave * per + per, nblk)
            for lane in range(64):
                i, q = lane & 15, lane >> 4
                n = wg * COLS + i
                blk = b0
                while blk < b1:
                    for j in range(batch):
                        if blk + j >= b1:
                            continue
                        for p in range(pc):
                            k = (blk + j) * kb + piece_k(dtype, q, p)
                            cnt = max(0, min(ue, K - k))
                            if n < N and cnt:
                                lo = n * ldb + k
                                assert 0 <= lo and lo + cnt <= b_end
                                for e in range(cnt):
                                    used[(n, k + e)] = used.get((n, k + e), 0) + 1
                            if i < M and cnt:
                                for e in range(cnt):
                                    off = (k + e) * lda + i if ta else i * lda + k + e
                                    assert 0 <= off < a_end
                    blk += batch
            # the reduction: wave 0's lane l writes C(l % 16, 16 wg + 4 (l / 16) + r)
        for lane in range(64):
            m, col = lane & 15, wg * COLS + 4 * (lane >> 4)
            if m >= M:
                continue
            for r in range(4):
                if col + r < N:
                    off = m * ldc + col + r
                    assert off <= (M - 1) * ldc + N - 1
                    written[(m, col + r)] = written.get((m, col + r), 0) + 1
    return used, written


SHAPES = [(1, 1, 1), (1, 16, 8), (3, 300, 5), (16, 33, 128), (9, 40, 1000), (5, 17, 4096 + 7),
          (2, 48, 257)]


@pytest.mark.parametrize("k", GEMV, ids=[k["name"] for k in GEMV])
def test_gemv_reads_cover_k_once_and_stay_inside(k):
    dtype, ta = k["dtype"], bool(k["transa"])
    assert k["transb"] == 1 and k["bk"] == fmt(dtype)[2]
    for (M, N, K), (pa, pb, pcc) in itertools.product(SHAPES, [(0, 0, 0), (3, 5, 2)]):
        lda, ldb, ldc = (M if ta else K) + pa, K + pb, N + pcc
        used, written = replay(dtype, ta, M, N, K, lda, ldb, ldc)
        assert set(used) == {(n, kk) for n in range(N) for kk in range(K)}, (M, N, K)
        assert set(used.values()) <= {1}
        assert set(written) == {(m, n) for m in range(M) for n in range(N)}
        assert set(written.values()) == {1}


def test_the_model_sees_a_lost_k():
    """A piece offset that skips k (16-bit lanes at 8q + 1) leaves k uncovered:
    the coverage check would fail."""
    global piece_k
    saved = piece_k
    try:
        piece_k = lambda dtype, q, p: 8 * q + 1  # noqa: E731
        used, _ = replay(sg.SGEMM_DTYPE_BF16, False, 1, 16, 64, 64, 64, 16)
        assert set(used) != {(n, kk) for n in range(16) for kk in range(64)}
    finally:
        piece_k = saved
