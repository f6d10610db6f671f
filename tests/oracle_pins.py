"""Pins for the CPU oracle: checks against facts fixed by mathematics.

Each pin takes a loaded oracle library (``lib``) and raises AssertionError on
a mismatch, so the same pins run against the real oracle and against mutants
with planted mistakes (tests/test_oracle_mutants.py).  None of them re-types
the oracle's loop: they use exact rational arithmetic, Python integers,
closed forms of special matrices, and invariants such as (AB)^T = B^T A^T.

What the oracle computes is C = alpha*A*B + beta*C for row-major FP32 operands
("GEMM 优化之路", problem statement), with beta == 0 meaning C is not read,
and the same product with A and B in bfloat16 or IEEE binary16 (the gsyq.cn
guide, section 5.1: 16-bit inputs, FP32 accumulation).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import oracle

U = 2.0 ** -53  # unit roundoff of FP64


def f32_of_fraction(q: Fraction) -> np.float32:
    """Round an exact rational to FP32, nearest-even, with no double rounding."""
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    # exponent e with 2**23 <= a / 2**e < 2**24
    e = a.numerator.bit_length() - a.denominator.bit_length() - 24
    while a / Fraction(2) ** e >= 2 ** 24:
        e += 1
    while a / Fraction(2) ** e < 2 ** 23:
        e -= 1
    e = max(e, -149)  # FP32 subnormal quantum
    scaled = a / Fraction(2) ** e
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return np.float32(sign * float(m) * 2.0 ** e)


def _dyadic(rng, shape, bits=24):
    """FP32 values exactly representable, in [-1, 1)."""
    return (2.0 * rng.random(shape, dtype=np.float32) - np.float32(1.0))


def _run(lib, A, B, C, alpha, beta, lda=None, ldb=None, ldc=None, with_t=True):
    M, K = A.shape
    N = B.shape[1]
    return oracle.gemm(M, N, K, alpha, A, lda or max(K, 1), B, ldb or max(N, 1),
                       beta, C, ldc or max(N, 1), with_t=with_t, lib=lib)


# --------------------------------------------------------------------------
def pin_bruteforce_exact(lib, seed=7, cases=60):
    """Random tiny problems against exact rational arithmetic.

    |r - exact| <= (K + 3) * 2**-53 * (|alpha| * t + |beta * c|), t matches the
    exact sum of |a*b| to K*2**-53 relative, and r rounded to FP32 equals the
    exact value rounded to FP32.  Covers both the full and the point modes.
    """
    rng = np.random.default_rng(seed)
    for case in range(cases):
        M, N, K = (int(x) for x in rng.integers(1, 9, size=3))
        alpha = float(rng.choice([1.0, 1.5, -0.75, 0.0, 2.0 ** -3]))
        beta = float(rng.choice([0.0, 0.5, 1.0, -1.25]))
        A = _dyadic(rng, (M, K))
        B = _dyadic(rng, (K, N))
        C = _dyadic(rng, (M, N))
        R, T = _run(lib, A, B, C, alpha, beta)
        rows = np.repeat(np.arange(M), N)
        cols = np.tile(np.arange(N), M)
        rp, tp = oracle.gemm_points(M, N, K, alpha, A, K, B, N, beta, C, N,
                                    rows, cols, lib=lib)
        qa, qb = Fraction(alpha), Fraction(beta)
        for i in range(M):
            for j in range(N):
                terms = [Fraction(float(A[i, k])) * Fraction(float(B[k, j]))
                         for k in range(K)]
                s = sum(terms, Fraction(0))
                t = sum((abs(x) for x in terms), Fraction(0))
                cterm = qb * Fraction(float(C[i, j])) if beta != 0 else Fraction(0)
                exact = qa * s + cterm
                scale = abs(alpha) * float(t) + abs(float(cterm))
                tol = (K + 3) * U * scale
                for r, tt, mode in ((R[i, j], T[i, j], "full"),
                                    (rp[i * N + j], tp[i * N + j], "points")):
                    err = abs(Fraction(float(r)) - exact)
                    assert err <= Fraction(tol) + Fraction(0), (
                        f"case {case} {mode} ({i},{j}) M,N,K={M},{N},{K}: "
                        f"err {float(err):.3e} > {tol:.3e}")
                    terr = abs(Fraction(float(tt)) - t)
                    assert terr <= Fraction(K * U * float(t)), (
                        f"case {case} {mode} t mismatch at ({i},{j})")
                    assert np.float32(r) == f32_of_fraction(exact), (
                        f"case {case} {mode} ({i},{j}): FP32 rounding differs")


def pin_integer_exact(lib, seed=11):
    """Integer inputs: every partial sum is exact, so r equals integer math."""
    rng = np.random.default_rng(seed)
    # small: Python ints, element by element
    M, N, K = 7, 5, 9
    A = rng.integers(-4, 5, (M, K))
    B = rng.integers(-4, 5, (K, N))
    C = rng.integers(-4, 5, (M, N))
    R, _ = _run(lib, A.astype(np.float32), B.astype(np.float32),
                C.astype(np.float32), 1.0, 1.0)
    for i in range(M):
        for j in range(N):
            want = sum(int(A[i, k]) * int(B[k, j]) for k in range(K)) + int(C[i, j])
            assert R[i, j] == want, f"({i},{j}) {R[i, j]} != {want}"
    # larger, several tiles' worth: int64 matrix product is exact
    M, N, K = 67, 45, 131
    A = rng.integers(-4, 5, (M, K))
    B = rng.integers(-4, 5, (K, N))
    C = rng.integers(-4, 5, (M, N))
    R, _ = _run(lib, A.astype(np.float32), B.astype(np.float32),
                C.astype(np.float32), 3.0, -2.0)
    want = 3 * (A.astype(np.int64) @ B.astype(np.int64)) - 2 * C
    assert np.array_equal(R, want.astype(np.float64))


def pin_identity(lib, seed=13):
    """A = I gives alpha*B + beta*C; B = I gives alpha*A + beta*C (exact here)."""
    rng = np.random.default_rng(seed)
    n, N = 19, 23
    alpha, beta = 1.5, 0.5
    B = _dyadic(rng, (n, N))
    C = _dyadic(rng, (n, N))
    R, _ = _run(lib, np.eye(n, dtype=np.float32), B, C, alpha, beta)
    assert np.array_equal(R, alpha * B.astype(np.float64) + beta * C.astype(np.float64))
    M = 17
    A = _dyadic(rng, (M, n))
    C2 = _dyadic(rng, (M, n))
    R, _ = _run(lib, A, np.eye(n, dtype=np.float32), C2, alpha, beta)
    assert np.array_equal(R, alpha * A.astype(np.float64) + beta * C2.astype(np.float64))


def pin_permutation(lib, seed=17):
    """A = P permutes the rows of B; B = P permutes the columns of A."""
    rng = np.random.default_rng(seed)
    n, N, M = 21, 13, 11
    perm = rng.permutation(n)
    P = np.zeros((n, n), dtype=np.float32)
    P[np.arange(n), perm] = 1.0  # (P B)[i] = B[perm[i]]
    B = _dyadic(rng, (n, N))
    C = np.full((n, N), np.nan, dtype=np.float32)
    R, _ = _run(lib, P, B, C, 1.0, 0.0)
    assert np.array_equal(R, B[perm].astype(np.float64))
    A = _dyadic(rng, (M, n))
    # (A P)[:, j] = sum_k A[:, k] P[k, j] = A[:, perm^-1[j]]
    R, _ = _run(lib, A, P, np.zeros((M, n), np.float32), -2.0, 0.0)
    inv = np.argsort(perm)
    assert np.array_equal(R, -2.0 * A[:, inv].astype(np.float64))


def pin_rank1(lib, seed=19):
    """K = 1: r = alpha*a_i*b_j + beta*c_ij; and A = u p^T, B = q w^T."""
    rng = np.random.default_rng(seed)
    M, N = 9, 14
    alpha, beta = 1.5, 0.5
    a = _dyadic(rng, (M, 1))
    b = _dyadic(rng, (1, N))
    C = _dyadic(rng, (M, N))
    R, _ = _run(lib, a, b, C, alpha, beta)
    want = alpha * (a.astype(np.float64) * b.astype(np.float64)) + beta * C.astype(np.float64)
    assert np.array_equal(R, want)
    # small-integer outer products: C_ij = alpha * u_i * (p . q) * w_j + beta * c_ij
    K = 33
    u = rng.integers(-3, 4, M)
    p = rng.integers(-3, 4, K)
    q = rng.integers(-3, 4, K)
    w = rng.integers(-3, 4, N)
    c = rng.integers(-3, 4, (M, N))
    A = np.outer(u, p).astype(np.float32)
    B = np.outer(q, w).astype(np.float32)
    R, _ = _run(lib, A, B, c.astype(np.float32), -1.0, 2.0)
    pq = int(np.dot(p, q))
    for i in range(M):
        for j in range(N):
            assert R[i, j] == -1 * int(u[i]) * pq * int(w[j]) + 2 * int(c[i, j])


def pin_alpha_beta(lib, seed=23):
    """alpha = 0 gives beta*C; beta = 0 never reads C; B = 0 with beta = 1 keeps C;
    K = 0 gives beta*C (zeros when beta = 0, even over a NaN C)."""
    rng = np.random.default_rng(seed)
    M, N, K = 6, 10, 12
    A = _dyadic(rng, (M, K))
    B = _dyadic(rng, (K, N))
    C = _dyadic(rng, (M, N))
    R, _ = _run(lib, A, B, C, 0.0, 0.5)
    assert np.array_equal(R, 0.5 * C.astype(np.float64))
    Cn = np.full((M, N), np.nan, dtype=np.float32)
    R1, _ = _run(lib, A, B, Cn, 1.0, 0.0)
    assert np.all(np.isfinite(R1))
    R2, _ = _run(lib, A, B, C, 1.0, 0.0)
    assert np.array_equal(R1, R2), "beta == 0 must not depend on C"
    R, _ = _run(lib, A, np.zeros((K, N), np.float32), C, 1.0, 1.0)
    assert np.array_equal(R, C.astype(np.float64))
    A0 = np.zeros((M, 0), np.float32)
    B0 = np.zeros((0, N), np.float32)
    R, _ = _run(lib, A0, B0, C, 1.0, -2.0)
    assert np.array_equal(R, -2.0 * C.astype(np.float64))
    R, _ = _run(lib, A0, B0, Cn, 1.0, 0.0)
    assert np.array_equal(R, np.zeros((M, N)))
    # alpha scales linearly: r(alpha=2^-3) == 2^-3 * r(alpha=1) exactly (power of 2)
    R8, _ = _run(lib, A, B, C, 0.125, 0.0)
    assert np.array_equal(R8, 0.125 * R2)


def pin_transpose(lib, seed=29):
    """(A B)^T = B^T A^T, bit for bit: the same products summed in the same order."""
    rng = np.random.default_rng(seed)
    M, N, K = 13, 7, 29
    A = _dyadic(rng, (M, K))
    B = _dyadic(rng, (K, N))
    R, T = _run(lib, A, B, None, 1.0, 0.0)
    Rt, Tt = _run(lib, np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), None, 1.0, 0.0)
    assert np.array_equal(R, Rt.T)
    assert np.array_equal(T, Tt.T)


def pin_leading_dims(lib, seed=31):
    """Padding beyond the M x N / M x K / K x N windows is never read (NaN pads)."""
    rng = np.random.default_rng(seed)
    M, N, K = 11, 9, 15
    alpha, beta = 1.5, 0.5
    A = _dyadic(rng, (M, K))
    B = _dyadic(rng, (K, N))
    C = _dyadic(rng, (M, N))
    R, T = _run(lib, A, B, C, alpha, beta)
    lda, ldb, ldc = K + 5, N + 3, N + 7

    def pad(x, ld):
        y = np.full((x.shape[0], ld), np.nan, np.float32)
        y[:, :x.shape[1]] = x
        return y

    Rp, Tp = oracle.gemm(M, N, K, alpha, pad(A, lda), lda, pad(B, ldb), ldb, beta,
                         pad(C, ldc), ldc, lib=lib)
    assert np.array_equal(R, Rp) and np.array_equal(T, Tp)
    rows = np.array([0, M - 1, 5, 3])
    cols = np.array([N - 1, 0, 4, 8])
    rp, tp = oracle.gemm_points(M, N, K, alpha, pad(A, lda), lda, pad(B, ldb), ldb,
                                beta, pad(C, ldc), ldc, rows, cols, lib=lib)
    assert np.array_equal(rp, R[rows, cols]) and np.array_equal(tp, T[rows, cols])


def pin_transposed_storage(lib, seed=37):
    """Storing A as A^T (K x M) or B as B^T (N x K) and setting the matching
    flag gives the untransposed result bit for bit (same products, same order);
    padding of the transposed storage is never read."""
    rng = np.random.default_rng(seed)
    M, N, K = 13, 11, 17
    alpha, beta = 1.5, 0.5
    A = _dyadic(rng, (M, K))
    B = _dyadic(rng, (K, N))
    C = _dyadic(rng, (M, N))
    R, T = _run(lib, A, B, C, alpha, beta)

    def pad(x, extra):
        y = np.full((x.shape[0], x.shape[1] + extra), np.nan, np.float32)
        y[:, :x.shape[1]] = x
        return y

    At = pad(np.ascontiguousarray(A.T), 3)  # K x (M+3)
    Bt = pad(np.ascontiguousarray(B.T), 5)  # N x (K+5)
    for ta, tb in ((True, False), (False, True), (True, True)):
        a, lda = (At, M + 3) if ta else (A, K)
        b, ldb = (Bt, K + 5) if tb else (B, N)
        R2, T2 = oracle.gemm(M, N, K, alpha, a, lda, b, ldb, beta, C, N, lib=lib,
                             ta=ta, tb=tb)
        assert np.array_equal(R, R2) and np.array_equal(T, T2), (ta, tb)
        rows, cols = np.array([0, 5, M - 1]), np.array([N - 1, 3, 0])
        rp, tp = oracle.gemm_points(M, N, K, alpha, a, lda, b, ldb, beta, C, N, rows,
                                    cols, lib=lib, ta=ta, tb=tb)
        assert np.array_equal(rp, R[rows, cols]) and np.array_equal(tp, T[rows, cols])


def pin_transposed_bruteforce(lib, seed=41, cases=12):
    """Transposed storage against exact rational sums on tiny problems."""
    rng = np.random.default_rng(seed)
    for case in range(cases):
        M, N, K = (int(x) for x in rng.integers(1, 7, size=3))
        ta, tb = bool(case & 1), bool(case & 2)
        A = _dyadic(rng, (M, K))
        B = _dyadic(rng, (K, N))
        a = np.ascontiguousarray(A.T) if ta else A
        b = np.ascontiguousarray(B.T) if tb else B
        R, _ = oracle.gemm(M, N, K, -0.75, a, M if ta else K, b, K if tb else N, 0.0,
                           None, N, lib=lib, ta=ta, tb=tb)
        for i in range(M):
            for j in range(N):
                exact = Fraction(-0.75) * sum(
                    (Fraction(float(A[i, k])) * Fraction(float(B[k, j])) for k in range(K)),
                    Fraction(0))
                assert abs(Fraction(float(R[i, j])) - exact) <= Fraction(
                    (K + 3) * U * 0.75 * float(sum(abs(Fraction(float(A[i, k])) *
                                                       Fraction(float(B[k, j])))
                                                   for k in range(K)))), (case, i, j)


# ---- 16-bit A and B (bfloat16, IEEE binary16), FP32 C ---------------------
#
# What the oracle decodes is fixed by the formats' definitions; the pins take
# the decoded values from library conversions (numpy's float16, torch's
# bfloat16), not from the oracle's own formulas.

F16_ONE = 0x3C00   # 1.0 in binary16
BF16_ONE = 0x3F80  # 1.0 in bfloat16


def values16(bits, dt):
    """FP64 values of 16-bit patterns by library conversion."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dt == "f16":
        return bits.view(np.float16).astype(np.float64)
    import torch
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()


def _same_values(got, want):
    both_nan = np.isnan(got) & np.isnan(want)
    return bool(np.all(both_nan | (got == want)))


def pin_lowp_decode(lib):
    """Every one of the 65536 patterns of each format, as an A element and as a
    B element (product with 1.0), equals the library conversion; NaN patterns
    give NaN, infinities infinities, binary16 subnormals their exact value."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for dt, one in (("bf16", BF16_ONE), ("f16", F16_ONE)):
        want = values16(allbits, dt)
        onev = np.array([one], np.uint16)
        R, _ = oracle.gemm_lowp(dt, 65536, 1, 1, 1.0, allbits, 1, onev, 1, 0.0, None,
                                1, with_t=False, lib=lib)
        assert _same_values(R[:, 0], want), f"{dt}: A-side decode differs"
        R, _ = oracle.gemm_lowp(dt, 1, 65536, 1, 1.0, onev, 1, allbits, 65536, 0.0,
                                None, 65536, with_t=False, lib=lib)
        assert _same_values(R[0, :], want), f"{dt}: B-side decode differs"
        # transposed storage reads the same patterns
        R, _ = oracle.gemm_lowp(dt, 65536, 1, 1, 1.0, allbits, 65536, onev, 1, 0.0,
                                None, 1, with_t=False, lib=lib, ta=True, tb=True)
        assert _same_values(R[:, 0], want), f"{dt}: transposed decode differs"


def _pattern_pair(rng, shape, dt):
    """Random finite 16-bit patterns of moderate magnitude and their values."""
    x = (2.0 * rng.random(shape) - 1.0).astype(np.float32)
    x *= np.float32(2.0) ** rng.integers(-12, 4, shape).astype(np.float32)
    from fp32_gemm_major_amd import workloads as wl
    bits = wl.round16(x, dt)
    return bits, values16(bits, dt).astype(np.float32)


def pin_lowp_matches_f32(lib, seed=43):
    """On values the 16-bit formats hold exactly, the 16-bit product equals
    the FP32 oracle's (itself pinned above) bit for bit, in both modes, for
    every storage, padded leading dimensions and alpha/beta."""
    rng = np.random.default_rng(seed)
    cases = [(5, 7, 9, 1.0, 0.0), (17, 3, 33, 1.5, 0.5), (1, 11, 4, -0.75, 1.0),
             (9, 1, 1, 2.0, -1.25), (6, 6, 0, 1.0, 0.5)]
    for dt in ("bf16", "f16"):
        for ci, (M, N, K, alpha, beta) in enumerate(cases):
            for ta in (False, True):
                for tb in (False, True):
                    a_bits, a_val = _pattern_pair(rng, (K, M) if ta else (M, K), dt)
                    b_bits, b_val = _pattern_pair(rng, (N, K) if tb else (K, N), dt)
                    C = _dyadic(rng, (M, N))
                    pa, pb = 2, 3  # padded leading dimensions
                    lda = (M if ta else K) + pa
                    ldb = (K if tb else N) + pb
                    A16 = np.zeros((a_bits.shape[0], lda), np.uint16)
                    A16[:, :a_bits.shape[1]] = a_bits
                    B16 = np.zeros((b_bits.shape[0], ldb), np.uint16)
                    B16[:, :b_bits.shape[1]] = b_bits
                    A32 = np.zeros(A16.shape, np.float32)
                    A32[:, :a_val.shape[1]] = a_val
                    B32 = np.zeros(B16.shape, np.float32)
                    B32[:, :b_val.shape[1]] = b_val
                    R16, T16 = oracle.gemm_lowp(dt, M, N, K, alpha, A16, lda, B16, ldb,
                                                beta, C, N, lib=lib, ta=ta, tb=tb)
                    R32, T32 = oracle.gemm(M, N, K, alpha, A32, lda, B32, ldb, beta,
                                           C, N, lib=lib, ta=ta, tb=tb)
                    tag = f"{dt} case {ci} ta={ta} tb={tb}"
                    assert np.array_equal(R16, R32), tag + ": r differs"
                    assert np.array_equal(T16, T32), tag + ": t differs"
                    if M and N:
                        rows = rng.integers(0, M, 8)
                        cols = rng.integers(0, N, 8)
                        rp, tp = oracle.gemm_lowp_points(dt, M, N, K, alpha, A16, lda,
                                                         B16, ldb, beta, C, N, rows,
                                                         cols, lib=lib, ta=ta, tb=tb)
                        assert np.array_equal(rp, R32[rows, cols]), tag + ": points r"
                        assert np.array_equal(tp, T32[rows, cols]), tag + ": points t"


def pin_lowp_bruteforce(lib, seed=47, cases=16):
    """Tiny 16-bit products, binary16 subnormals and bfloat16 extremes
    included, against exact rational sums of the library-decoded values."""
    rng = np.random.default_rng(seed)
    for case in range(cases):
        dt = "f16" if case % 2 else "bf16"
        M, N, K = (int(x) for x in rng.integers(1, 6, size=3))
        if dt == "f16":
            # any finite pattern: exponent field 0..30 (subnormals included)
            a_bits = rng.integers(0, 0x7C00, (M, K)).astype(np.uint16)
            b_bits = rng.integers(0, 0x7C00, (K, N)).astype(np.uint16)
        else:
            # exponent fields 0x20..0xDF keep every product and sum finite
            a_bits = rng.integers(0x1000, 0x7000, (M, K)).astype(np.uint16)
            b_bits = rng.integers(0x1000, 0x7000, (K, N)).astype(np.uint16)
        a_bits |= (rng.integers(0, 2, a_bits.shape) << 15).astype(np.uint16)
        b_bits |= (rng.integers(0, 2, b_bits.shape) << 15).astype(np.uint16)
        av, bv = values16(a_bits, dt), values16(b_bits, dt)
        R, _ = oracle.gemm_lowp(dt, M, N, K, 1.0, a_bits, K, b_bits, N, 0.0, None, N,
                                lib=lib)
        for i in range(M):
            for j in range(N):
                terms = [Fraction(float(av[i, k])) * Fraction(float(bv[k, j]))
                         for k in range(K)]
                exact = sum(terms, Fraction(0))
                t = float(sum((abs(x) for x in terms), Fraction(0)))
                err = abs(Fraction(float(R[i, j])) - exact)
                assert err <= Fraction((K + 3) * U * t), (dt, case, i, j)


# ---- 8-bit A and B (OCP E4M3, E5M2), FP32 C ---------------------------------

FP8_ONE = {"fp8e4m3": 0x38, "fp8e5m2": 0x3C}  # 1.0


def values8(bits, dt):
    """FP64 values of 8-bit patterns by torch's conversions."""
    import torch
    tdt = {"fp8e4m3": torch.float8_e4m3fn, "fp8e5m2": torch.float8_e5m2}[dt]
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    return torch.from_numpy(bits).view(tdt).double().numpy()


def pin_fp8_decode(lib):
    """All 256 patterns of each 8-bit format, as an A element and as a B
    element (product with 1.0), and in transposed storage, equal torch's
    conversions (NaN for NaN, infinities for E5M2's)."""
    allbits = np.arange(256, dtype=np.uint32).astype(np.uint8)
    for dt, one in FP8_ONE.items():
        want = values8(allbits, dt)
        onev = np.array([one], np.uint8)
        R, _ = oracle.gemm_lowp(dt, 256, 1, 1, 1.0, allbits, 1, onev, 1, 0.0, None, 1,
                                with_t=False, lib=lib)
        assert _same_values(R[:, 0], want), f"{dt}: A-side decode differs"
        R, _ = oracle.gemm_lowp(dt, 1, 256, 1, 1.0, onev, 1, allbits, 256, 0.0, None, 256,
                                with_t=False, lib=lib)
        assert _same_values(R[0, :], want), f"{dt}: B-side decode differs"
        R, _ = oracle.gemm_lowp(dt, 256, 1, 1, 1.0, allbits, 256, onev, 1, 0.0, None, 1,
                                with_t=False, lib=lib, ta=True, tb=True)
        assert _same_values(R[:, 0], want), f"{dt}: transposed decode differs"


def pin_fp8_matches_f32(lib, seed=53):
    """On values the 8-bit formats hold exactly, the 8-bit product equals the
    FP32 oracle's bit for bit (full and point modes, every storage, padded
    leading dimensions)."""
    from fp32_gemm_major_amd import workloads as wl
    rng = np.random.default_rng(seed)
    for dt in wl.FORMATS8:
        for ci, (M, N, K, alpha, beta) in enumerate([(5, 7, 9, 1.0, 0.0),
                                                     (13, 4, 21, 1.5, 0.5),
                                                     (3, 11, 1, -2.0, 1.0)]):
            for ta in (False, True):
                for tb in (False, True):
                    def operand(rows, cols):
                        x = (2.0 * rng.random((rows, cols)) - 1.0).astype(np.float32)
                        x *= np.float32(2.0) ** rng.integers(-6, 4, (rows, cols)).astype(np.float32)
                        bits = wl.round8(x, dt)
                        buf = np.zeros((rows, cols + 3), np.uint8)
                        buf[:, :cols] = bits
                        val = np.zeros((rows, cols + 3), np.float32)
                        val[:, :cols] = values8(bits, dt)
                        return buf, val
                    A8, A32 = operand(*((K, M) if ta else (M, K)))
                    B8, B32 = operand(*((N, K) if tb else (K, N)))
                    C = _dyadic(rng, (M, N))
                    lda, ldb = A8.shape[1], B8.shape[1]
                    R8, T8 = oracle.gemm_lowp(dt, M, N, K, alpha, A8, lda, B8, ldb, beta, C,
                                              N, lib=lib, ta=ta, tb=tb)
                    R32, T32 = oracle.gemm(M, N, K, alpha, A32, lda, B32, ldb, beta, C, N,
                                           lib=lib, ta=ta, tb=tb)
                    tag = f"{dt} case {ci} ta={ta} tb={tb}"
                    assert np.array_equal(R8, R32) and np.array_equal(T8, T32), tag
                    rows, cols = rng.integers(0, M, 6), rng.integers(0, N, 6)
                    rp, tp = oracle.gemm_lowp_points(dt, M, N, K, alpha, A8, lda, B8, ldb,
                                                     beta, C, N, rows, cols, lib=lib,
                                                     ta=ta, tb=tb)
                    assert np.array_equal(rp, R32[rows, cols]), tag + " points"
                    assert np.array_equal(tp, T32[rows, cols]), tag + " points t"


def pin_fp8_bruteforce(lib, seed=59, cases=12):
    """Tiny 8-bit products over every finite pattern class (subnormals
    included) against exact rational sums of torch-decoded values."""
    rng = np.random.default_rng(seed)
    for case in range(cases):
        dt = "fp8e5m2" if case % 2 else "fp8e4m3"
        M, N, K = (int(x) for x in rng.integers(1, 6, size=3))
        top = 0x7E if dt == "fp8e4m3" else 0x7B   # largest finite magnitude
        a_bits = rng.integers(0, top + 1, (M, K)).astype(np.uint8)
        b_bits = rng.integers(0, top + 1, (K, N)).astype(np.uint8)
        a_bits |= (rng.integers(0, 2, a_bits.shape) << 7).astype(np.uint8)
        b_bits |= (rng.integers(0, 2, b_bits.shape) << 7).astype(np.uint8)
        av, bv = values8(a_bits, dt), values8(b_bits, dt)
        R, _ = oracle.gemm_lowp(dt, M, N, K, 1.0, a_bits, K, b_bits, N, 0.0, None, N,
                                lib=lib)
        for i in range(M):
            for j in range(N):
                terms = [Fraction(float(av[i, k])) * Fraction(float(bv[k, j]))
                         for k in range(K)]
                exact = sum(terms, Fraction(0))
                t = float(sum((abs(x) for x in terms), Fraction(0)))
                assert abs(Fraction(float(R[i, j])) - exact) <= Fraction((K + 3) * U * t), \
                    (dt, case, i, j)


ALL_PINS = [pin_bruteforce_exact, pin_integer_exact, pin_identity,
            pin_permutation, pin_rank1, pin_alpha_beta, pin_transpose,
            pin_leading_dims, pin_transposed_storage, pin_transposed_bruteforce,
            pin_lowp_decode, pin_lowp_matches_f32, pin_lowp_bruteforce,
            pin_fp8_decode, pin_fp8_matches_f32, pin_fp8_bruteforce]
