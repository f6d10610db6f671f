"""CPU model of the one-pass small-M FP32 kernels (skinny_sgemm.hpp):
skinny_nt_kernel (B stored N x K) and skinny_kn_kernel (B stored K x N).

The kernel's index arithmetic, replayed per wave and lane for a range of
shapes, leading dimensions and both storages of A:

* every element it loads lies inside the operand windows the C ABI
  validates (rows past N and M clamped to the last one, the last piece of K
  read from clamped addresses);
* every k of every row of B is multiplied exactly once with the same k of
  every row of A, and nothing past K contributes;
* every output (m < M, n < N) is written exactly once and nothing else is;
* the recursive halving leaves, in the lane the kernel reads it from, the
  exact sum over the 64 lanes of each partial sum (integers, so any
  misrouted or twice-counted lane shows).
"""
import itertools

import numpy as np
import pytest

import fp32_gemm_major_amd as sg

KERNELS = sg.kernel_table() if __import__("os").path.exists(sg.LIBRARY) else []
ONE_PASS = [k for k in KERNELS if k["schedule"] == sg.SGEMM_SCHEDULE_SMALL_M
            and k["variant"] == sg.SGEMM_VARIANT_VALU and k["transb"]]

WAVES, PIECE = 8, 256


def rows_per_workgroup(mt):
    return 8 if mt <= 2 else 4


def load16(n_left):
    """Offsets (within the 16 bytes) that a lane's load reads, and which of
    them hold data: the kernel's whole load, or the clamped partial one."""
    if n_left >= 4:
        return [0, 1, 2, 3], [True] * 4
    if n_left <= 0:
        return [], []
    return [e if e < n_left else n_left - 1 for e in range(4)], [e < n_left for e in range(4)]


def replay(mt, ta, M, N, K, lda, ldb, ldc):
    R = rows_per_workgroup(mt)
    a_end = ((K - 1) * lda + M) if ta else ((M - 1) * lda + K)  # elements
    b_end = (N - 1) * ldb + K
    used = {}
    written = {}
    np_ = K // PIECE + (K % PIECE != 0)
    per = -(-np_ // WAVES)
    for wg in range(-(-N // R)):
        n0 = wg * R
        brow = [min(n0 + r, N - 1) for r in range(R)]
        am = [min(m, M - 1) for m in range(mt)]
        for wave in range(WAVES):
            p0, p1 = wave * per, min(wave * per + per, np_)
            for p in range(p0, p1):
                whole = (p + 1) * PIECE <= K
                for lane in range(64):
                    k = p * PIECE + 4 * lane
                    offs, live = ([0, 1, 2, 3], [True] * 4) if whole else load16(K - k)
                    for r in range(R):
                        for e, ok in zip(offs, live):
                            addr = brow[r] * ldb + k + e
                            assert 0 <= addr < b_end, (wg, wave, lane, r)
                    for m in range(mt):
                        for e, ok in zip(offs, live):
                            addr = (k + e) * lda + am[m] if ta else am[m] * lda + k + e
                            assert 0 <= addr < a_end, (wg, wave, lane, m)
                    # products that reach a stored sum: element e of the
                    # lane's B piece (masked to zero when not live) times the
                    # same element of the A piece
                    for e in range(4):
                        if whole or (e < len(live) and live[e]):
                            kk = k + e
                            assert kk < K
                            for r in range(R):
                                n = n0 + r
                                if n >= N:
                                    continue
                                for m in range(M):
                                    used[(m, n, kk)] = used.get((m, n, kk), 0) + 1
        for t in range(mt * R):
            m, r = t // R, t % R
            if m < M and n0 + r < N:
                off = m * ldc + n0 + r
                written[off] = written.get(off, 0) + 1
    assert len(used) == M * N * K and set(used.values()) == {1}
    want = {m * ldc + n for m in range(M) for n in range(N)}
    assert set(written) == want and set(written.values()) == {1}


def halving(vals):
    """The kernel's reduction over 64 lanes of V sums each: returns what each
    lane holds in acc[0] at the end."""
    V = vals.shape[1]
    acc = [list(vals[l]) for l in range(64)]
    cnt = V
    off = 32
    while off >= 1:
        new = [a[:] for a in acc]
        for l in range(64):
            up = (l & off) != 0
            partner = acc[l ^ off]
            if cnt > 1:
                half = cnt // 2
                for i in range(half):
                    # the partner sends the half this lane keeps
                    send = partner[i] if (l ^ off) & off else partner[i + half]
                    keep = acc[l][i + half] if up else acc[l][i]
                    new[l][i] = keep + send
            else:
                new[l][0] = acc[l][0] + partner[0]
        acc = new
        if cnt > 1:
            cnt //= 2
        off //= 2
    return [a[0] for a in acc]


@pytest.mark.parametrize("V", [1, 2, 4, 8, 16, 32, 64])
def test_recursive_halving_sums(V):
    rng = np.random.default_rng(V)
    vals = rng.integers(-1000, 1000, size=(64, V))
    out = halving(vals)
    logv = V.bit_length() - 1
    want = vals.sum(axis=0)
    for lane in range(64):
        if lane & ((64 >> logv) - 1) == 0:
            assert out[lane] == want[lane >> (6 - logv)], (V, lane)


def test_halving_catches_a_wrong_keep():
    """A halving step that keeps the wrong half (the mistake the bitwise
    select could make) does not give the sums."""
    V = 8
    vals = np.random.default_rng(1).integers(-1000, 1000, size=(64, V))
    acc = [list(vals[l]) for l in range(64)]
    cnt, off = V, 32
    while off >= 1:
        new = [a[:] for a in acc]
        for l in range(64):
            partner = acc[l ^ off]
            if cnt > 1:
                half = cnt // 2
                for i in range(half):
                    up = (l & off) != 0
                    send = partner[i] if (l ^ off) & off else partner[i + half]
                    keep = acc[l][i] if up else acc[l][i + half]   # swapped
                    new[l][i] = keep + send
            else:
                new[l][0] = acc[l][0] + partner[0]
        acc = new
        cnt = max(1, cnt // 2)
        off //= 2
    want = vals.sum(axis=0)
    assert any(acc[l][0] != want[l >> 3] for l in range(0, 64, 8))


def test_table_matches_model():
    if not KERNELS:
        pytest.skip("library not built")
    assert sorted((k["bm"], k["transa"]) for k in ONE_PASS) == \
        sorted((m, a) for m in (1, 2, 4, 8) for a in (0, 1))
    for k in ONE_PASS:
        assert k["bn"] == rows_per_workgroup(k["bm"]) and k["threads"] == 64 * WAVES
        assert k["bk"] == PIECE


SHAPES = [(1, 1, 1), (1, 9, 255), (2, 8, 256), (3, 5, 257), (4, 13, 300),
          (8, 7, 2049), (5, 4, 4 * 256 + 3), (7, 17, 9 * 256)]


@pytest.mark.parametrize("mt,ta", list(itertools.product((1, 2, 4, 8), (False, True))))
def test_reads_in_bounds_and_cover_k_once(mt, ta):
    for M, N, K in SHAPES:
        M = min(M, mt)
        for pad in (0, 3):
            lda = (M if ta else K) + pad
            replay(mt, ta, M, N, K, lda, K + pad, N + pad)


# ---- B stored K x N (skinny_kn_kernel) -------------------------------------

KN_WAVES, KN_COLS = 16, 32
KN_LPR = KN_COLS // 4
KN_RG = 64 // KN_LPR
KN_UNIT = 4 * KN_RG
KN_TABLE = [k for k in KERNELS if k["schedule"] == sg.SGEMM_SCHEDULE_SMALL_M
            and k["variant"] == sg.SGEMM_VARIANT_VALU and not k["transb"] and k["bn"] == KN_COLS]


def replay_kn(mt, ta, M, N, K, lda, ldb, ldc):
    batch = 2 if mt == 1 else 1
    a_end = ((K - 1) * lda + M) if ta else ((M - 1) * lda + K)
    b_end = (K - 1) * ldb + N
    used = {}
    written = {}
    nu = K // KN_UNIT + (K % KN_UNIT != 0)
    per = -(-nu // KN_WAVES)
    am = [min(m, M - 1) for m in range(mt)]
    for wg in range(-(-N // KN_COLS)):
        n0 = wg * KN_COLS
        cols_whole = n0 + KN_COLS <= N
        for wave in range(KN_WAVES):
            u0, u1 = wave * per, min(wave * per + per, nu)
            u = u0
            while u < u1:
                whole = cols_whole and u + batch <= u1 and (u + batch) * KN_UNIT <= K
                for t in range(batch):
                    for lane in range(64):
                        cg, rg = lane % KN_LPR, lane // KN_LPR
                        n = n0 + 4 * cg
                        ncl = min(n, N - 1)
                        k = (u + t) * KN_UNIT + 4 * rg
                        if whole:
                            kleft, cols = 4, [(n + e, True) for e in range(4)]
                        else:
                            kleft = K - k if u + t < u1 else 0
                            offs, live = load16(N - n)
                            cols = [(ncl + o, ok) for o, ok in zip(offs, live)]
                        rows = [k + j for j in range(4) if j < kleft]
                        for kk in rows:
                            for col, ok in cols:
                                assert 0 <= kk * ldb + col < b_end, (wg, wave, lane)
                        a_offs, a_live = ([0, 1, 2, 3], [True] * 4) if whole else load16(kleft)
                        kb = k if (whole or kleft > 0) else 0
                        for m in range(mt):
                            for o in a_offs:
                                addr = (kb + o) * lda + am[m] if ta else am[m] * lda + kb + o
                                assert 0 <= addr < a_end, (wg, wave, lane, m)
                        for j, kk in enumerate(rows):
                            if not (whole or a_live[j]):
                                continue
                            for e, (col, ok) in enumerate(cols if whole else
                                                          [(n + e, e < len(cols) and cols[e][1])
                                                           for e in range(4)]):
                                if not ok or n + e >= N:
                                    continue
                                for m in range(M):
                                    key = (m, n + e, kk)
                                    used[key] = used.get(key, 0) + 1
                u += batch
        for t in range(KN_LPR * mt * 4):
            c, v = t // (mt * 4), t % (mt * 4)
            m, col = v // 4, n0 + 4 * c + v % 4
            if m < M and col < N:
                off = m * ldc + col
                written[off] = written.get(off, 0) + 1
    assert len(used) == M * N * K and set(used.values()) == {1}
    want = {m * ldc + n for m in range(M) for n in range(N)}
    assert set(written) == want and set(written.values()) == {1}


def halving_kn(vals, lpr):
    """The K x N kernel's reduction: recursive halving over the lane bits at
    and above lpr (the row groups); returns, per lane, the sums it holds and
    the index of the first."""
    V = vals.shape[1]
    acc = [list(vals[l]) for l in range(64)]
    base = [0] * 64
    cnt, off = V, 32
    while off >= lpr:
        new = [a[:] for a in acc]
        for l in range(64):
            up = (l & off) != 0
            partner = acc[l ^ off]
            if cnt > 1:
                half = cnt // 2
                for i in range(half):
                    send = partner[i] if (l ^ off) & off else partner[i + half]
                    keep = acc[l][i + half] if up else acc[l][i]
                    new[l][i] = keep + send
                if up:
                    base[l] += half
            else:
                new[l][0] = acc[l][0] + partner[0]
        acc = new
        if cnt > 1:
            cnt //= 2
        off //= 2
    return [(a[:cnt], b) for a, b in zip(acc, base)]


@pytest.mark.parametrize("mt", [1, 2, 4, 8])
def test_kn_halving_sums(mt):
    V = 4 * mt
    halve = min(V.bit_length() - 1, 3)
    rng = np.random.default_rng(mt)
    vals = rng.integers(-1000, 1000, size=(64, V))
    out = halving_kn(vals, KN_LPR)
    seen = set()
    for lane in range(64):
        cg, rg = lane % KN_LPR, lane // KN_LPR
        if rg & ((1 << (3 - halve)) - 1):
            continue  # not a writer
        sums, base = out[lane]
        assert len(sums) == V >> halve
        for i, x in enumerate(sums):
            col_lanes = [l for l in range(64) if l % KN_LPR == cg]
            assert x == sum(vals[l][base + i] for l in col_lanes), (mt, lane, i)
            assert (cg, base + i) not in seen
            seen.add((cg, base + i))
    assert seen == {(c, v) for c in range(KN_LPR) for v in range(V)}


def test_kn_table_matches_model():
    if not KERNELS:
        pytest.skip("library not built")
    assert sorted((k["bm"], k["transa"]) for k in KN_TABLE) == \
        sorted((m, a) for m in (1, 2, 4, 8) for a in (0, 1))
    for k in KN_TABLE:
        assert (k["bk"], k["threads"]) == (KN_UNIT, 64 * KN_WAVES)


KN_SHAPES = [(1, 1, 1), (1, 33, 31), (2, 32, 32), (3, 37, 33), (4, 64, 300),
             (4, 31, 513), (2, 70, 16 * 32 + 5), (1, 5, 2 * 16 * 32 + 64), (8, 40, 777),
             (7, 33, 65)]


@pytest.mark.parametrize("mt,ta", list(itertools.product((1, 2, 4, 8), (False, True))))
def test_kn_reads_in_bounds_and_cover_k_once(mt, ta):
    for M, N, K in KN_SHAPES:
        M = min(M, mt)
        for pad in (0, 3):
            lda = (M if ta else K) + pad
            replay_kn(mt, ta, M, N, K, lda, N + pad, N + pad)
