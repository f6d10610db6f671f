"""Pins for the acceptance bound of the parity tests, ``oracle.error_bound``.

The bound is, elementwise against the unrounded result r,

    |C - r| <= 4 * max(K, 1) * 2**-24 * (|alpha| * t + |beta * c|),

with t = sum_k |a_ik * b_kj| and the beta term 0 when beta == 0 (C is then
not read and may hold NaN).  It is the a-priori bound of a length-K FP32 dot
product in any order of the additions (Higham, "Accuracy and Stability of
Numerical Algorithms", section 3.1: |fl(x.y) - x.y| <= gamma_K |x|.|y| with
gamma_K = K*u / (1 - K*u), u = 2**-24), widened to cover the roundings of the
alpha/beta update.  The pages themselves give three tolerances that do not
agree ("GEMM 优化之路", complete listing's check; the T4 article's relative
1e-3; the gsyq.cn guide, section 6.1's relative 1e-5), so this one replaces
them.

Every pin takes the bound as a function argument, so the same pins run
against planted mistakes in it (tests/test_oracle_mutants.py).  None of them
re-types the formula to compare against itself; they hold it to what FP32
arithmetic does:

- it admits every legitimate FP32 evaluation: dot products accumulated with
  IEEE single-precision operations on the CPU (numpy float32 arithmetic is
  correctly rounded) in several orders -- sequential, pairwise, blocks of 32,
  fused multiply-add -- with the alpha/beta update in two orders, on random,
  one-signed, cancelling and adversarial inputs, K from 0 to 4096; some of
  these are built to reach well over half the bound, so a bound that is too
  tight by a factor of two fails;
- it rejects results computed from inputs held with a 10-bit mantissa (the
  input precision of binary16 or a TF32-style path) on inputs built to show
  that loss, at the K where the true bound still can (K < 2047 for this
  construction), so a bound that is too loose by a factor of two, or that
  grows as K*K, fails;
- it gives the values worked out by hand in tests/golden/error_bound.json.

The exact result r is taken in FP64 from exactly computed products (a
product of two FP32 values is exact in FP64) summed by ``math.fsum``
(correctly rounded), so it is within a few units of 2**-53 of the exact
value; every comparison below widens or narrows by that margin in the
direction that keeps the pin sound.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

F32 = np.float32
U = 2.0 ** -24
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "error_bound.json")


# ---- exact sums and FP32 evaluations (independent of the oracle) -----------

def _exact(a_row, b_col, alpha, beta, c):
    """(r, t, margin) for one output: r = alpha*sum(a*b) + beta*c and
    t = sum|a*b| in FP64 from exact products and fsum; ``margin`` bounds
    |r - exact| (a few 2**-53 roundings of the scale)."""
    prods = [float(x) * float(y) for x, y in zip(a_row, b_col)]  # exact in FP64
    s = math.fsum(prods)
    t = math.fsum(abs(p) for p in prods)
    cterm = float(beta) * float(c) if beta != 0 else 0.0
    r = float(alpha) * s + cterm
    scale = abs(float(alpha)) * t + abs(cterm)
    return r, t, 8.0 * 2.0 ** -53 * scale


def _dot_sequential(p):
    s = np.zeros(p.shape[1:], F32)
    for k in range(p.shape[0]):
        s = F32(s + p[k])
    return s


def _dot_pairwise(p):
    x = p
    if x.shape[0] == 0:
        return np.zeros(p.shape[1:], F32)
    while x.shape[0] > 1:
        if x.shape[0] % 2:
            x = np.concatenate([x, np.zeros((1,) + x.shape[1:], F32)])
        x = F32(x[0::2] + x[1::2])
    return x[0]


def _dot_blocked(p, block=32):
    parts = [_dot_sequential(p[k:k + block]) for k in range(0, p.shape[0], block)]
    return _dot_sequential(np.stack(parts)) if parts else np.zeros(p.shape[1:], F32)


def _dot_fused(a, b):
    """s <- fl32(a_k*b_k + s): the product is exact in FP64; the FP64 sum can
    round once before the FP32 rounding, which moves a result only at an
    FP32 tie (still within one FP32 rounding plus 2**-53 relative)."""
    s = np.zeros((a.shape[0], b.shape[1]), np.float64)
    for k in range(a.shape[1]):
        s = (a[:, k:k + 1].astype(np.float64) * b[k:k + 1, :].astype(np.float64)
             + s).astype(F32).astype(np.float64)
    return s.astype(F32)


def _products(a, b):
    """FP32-rounded products, shape (K, M, N)."""
    return F32(a.T[:, :, None] * b[:, None, :])


def _update(s, alpha, beta, c, order):
    """The alpha/beta update in FP32: two roundings and a sum, or a fused
    alpha*s + fl32(beta*c)."""
    cterm = F32(F32(beta) * c) if beta != 0 else np.zeros_like(s)
    if order == "separate":
        return F32(F32(F32(alpha) * s) + cterm)
    return (np.float64(alpha) * s.astype(np.float64) + cterm.astype(np.float64)).astype(F32)


def _exact_all(a, b, alpha, beta, c):
    """_exact for every output of an M x N problem: (R, T, MARGIN)."""
    M, N = a.shape[0], b.shape[1]
    R, T, G = (np.zeros((M, N)) for _ in range(3))
    for i in range(M):
        for j in range(N):
            R[i, j], T[i, j], G[i, j] = _exact(a[i], b[:, j], alpha, beta, c[i, j])
    return R, T, G


def _ratio_of(bound, K, alpha, beta, c, out, exact):
    """max over outputs of (|out - r| + margin) / bound, given _exact_all's
    (R, T, MARGIN)."""
    R, T, G = exact
    bd = np.asarray(bound(K, alpha, beta, T, c.astype(np.float64)), np.float64)
    err = np.abs(out.astype(np.float64) - R) + G
    exact_out = (err == G) & (err <= bd)
    if np.any(~exact_out & ~(bd > 0)):
        return math.inf
    ratio = np.where(exact_out, 0.0, err / np.where(bd > 0, bd, 1.0))
    return float(ratio.max()) if ratio.size else 0.0


# ---- pins --------------------------------------------------------------------

def pin_bound_admits_fp32_orders(bound, seed=31):
    """FP32 dot products in four orders and the update in two orders, on
    random, one-signed and small-normal inputs, K up to 4096, and alpha/beta
    of both signs (a NaN C with beta = 0 included): all within the bound."""
    rng = np.random.default_rng(seed)
    M, N = 4, 5
    for K in (1, 2, 3, 7, 64, 777, 4096):
        for dist in ("uniform", "positive", "normal"):
            if dist == "uniform":
                a = F32(2 * rng.random((M, K), dtype=F32) - 1)
                b = F32(2 * rng.random((K, N), dtype=F32) - 1)
            elif dist == "positive":
                a = rng.random((M, K), dtype=F32)
                b = rng.random((K, N), dtype=F32)
            else:
                a = F32(rng.standard_normal((M, K), dtype=F32) * F32(0.02))
                b = F32(rng.standard_normal((K, N), dtype=F32) * F32(0.02))
            for alpha, beta in ((1.5, 0.5), (-0.75, 0.0), (1.0, -1.25), (F32(0.1), F32(0.3))):
                c = F32(2 * rng.random((M, N), dtype=F32) - 1)
                if beta == 0:
                    c = np.full((M, N), np.nan, F32)
                p = _products(a, b)
                exact = _exact_all(a, b, alpha, beta, c)
                sums = [_dot_sequential(p), _dot_pairwise(p), _dot_blocked(p), _dot_fused(a, b)]
                for s in sums:
                    for order in ("separate", "fused"):
                        out = _update(s, alpha, beta, c, order)
                        ratio = _ratio_of(bound, K, alpha, beta, c, out, exact)
                        assert ratio <= 1.0, (K, dist, alpha, beta, order, ratio)


def pin_bound_admits_adversarial_sums(bound):
    """Inputs where FP32 evaluation loses the most.

    Sequential sums of 1 and K-1 terms just under half an ulp of 1: every
    addition rounds back to 1, so the error is (K-1)*(2**-24 - 2**-34), about
    K*u*t (a quarter of the bound): a bound growing as sqrt(K) fails this.
    Cancelling sums (1, a term under half an ulp, -1): error about u*t/2
    against an exact result near 0, so a bound scaled by |r| instead of t
    fails.  Both must pass the true bound."""
    delta = F32(2.0 ** -24 - 2.0 ** -34)
    for K in (2, 3, 17, 256, 4096):
        a = np.full((1, K), delta, F32)
        a[0, 0] = 1.0
        b = np.ones((K, 1), F32)
        out = _update(_dot_sequential(_products(a, b)), 1.0, 0.0, np.zeros((1, 1), F32),
                      "separate")
        assert out[0, 0] == 1.0  # every small term lost, as constructed
        c0 = np.zeros((1, 1), F32)
        ratio = _ratio_of(bound, K, 1.0, 0.0, c0, out, _exact_all(a, b, 1.0, 0.0, c0))
        assert 0.9 * (K - 1) / (4 * K) < ratio <= 1.0, (K, ratio)
    a = np.array([[1.0, delta, -1.0]], F32)
    b = np.ones((3, 1), F32)
    out = _update(_dot_sequential(_products(a, b)), 1.0, 0.0, np.zeros((1, 1), F32),
                  "separate")
    assert out[0, 0] == 0.0  # exact result delta, computed 0
    c0 = np.zeros((1, 1), F32)
    ratio = _ratio_of(bound, 3, 1.0, 0.0, c0, out, _exact_all(a, b, 1.0, 0.0, c0))
    assert ratio <= 1.0, ratio


def _k1_stress_cases(seed, want=24):
    """K = 1 problems whose FP32 evaluation fl(fl(alpha*fl(a*b)) + fl(beta*c))
    errs the most relative to |alpha*a*b| + |beta*c|: found by a seeded search,
    ranked by an FP64 estimate and then measured exactly (Fractions)."""
    rng = np.random.default_rng(seed)
    n = 200000
    a = F32(1 + rng.random(n, dtype=F32))
    b = F32(1 + rng.random(n, dtype=F32))
    alpha = F32(1 + rng.random(n, dtype=F32)) * F32(np.where(rng.random(n) < 0.5, -1, 1))
    beta = F32(rng.random(n, dtype=F32) * F32(2.0 ** -12))
    c = F32(1 + rng.random(n, dtype=F32))
    p = F32(a * b)
    out = F32(F32(alpha * p) + F32(beta * c))
    est = (np.abs(out.astype(np.float64) - (alpha.astype(np.float64) * a * b + beta.astype(np.float64) * c))
           / (np.abs(alpha.astype(np.float64) * a * b) + np.abs(beta.astype(np.float64) * c)))
    idx = np.argsort(est)[-want:]
    cases = []
    for i in idx:
        exact = (Fraction(float(alpha[i])) * Fraction(float(a[i])) * Fraction(float(b[i]))
                 + Fraction(float(beta[i])) * Fraction(float(c[i])))
        scale = (abs(Fraction(float(alpha[i])) * Fraction(float(a[i])) * Fraction(float(b[i])))
                 + abs(Fraction(float(beta[i])) * Fraction(float(c[i]))))
        err = abs(Fraction(float(out[i])) - exact)
        cases.append((float(a[i]), float(b[i]), float(alpha[i]), float(beta[i]), float(c[i]),
                      err, scale))
    return cases


def pin_bound_admits_k1_update(bound):
    """K = 1 with all four roundings of the update (product, alpha scale, beta
    scale, sum) in play: the worst cases of a seeded search err by more than
    twice 2**-24 of the scale, so a bound too tight by two fails; the true
    bound (4 * 2**-24 * scale) admits them, checked in exact arithmetic."""
    cases = _k1_stress_cases(37)
    worst_rel = max(float(err / scale) for *_, err, scale in cases)
    assert worst_rel > 2.0 * U, worst_rel  # the search found real stress cases
    for a, b, alpha, beta, c, err, scale in cases:
        t = abs(a * b)  # exact in FP64
        bd = Fraction(float(np.asarray(bound(1, alpha, beta, np.float64(t), np.float64(c)))))
        assert err <= bd, (a, b, alpha, beta, c, float(err), float(bd))


def pin_bound_beta_and_empty_k(bound, seed=41):
    """C = fl32(beta*c) when alpha*A*B contributes nothing (K = 0, or
    alpha = 0): the one rounding of beta*c must be admitted, so the bound
    keeps its beta term and its floor of one term at K = 0; with beta = 0 a
    NaN C leaves the bound finite."""
    rng = np.random.default_rng(seed)
    c = F32(2 * rng.random(64, dtype=F32) - 1)
    beta = F32(0.1)
    got = F32(beta * c)
    exact = [Fraction(float(beta)) * Fraction(float(x)) for x in c]
    rounded = [Fraction(float(g)) != e for g, e in zip(got, exact)]
    assert sum(rounded) > 32  # most of these products do round
    for K, alpha in ((0, 1.0), (5, 0.0)):
        for x, g, e in zip(c, got, exact):
            bd = Fraction(float(np.asarray(bound(K, alpha, float(beta), np.float64(0.0),
                                                 np.float64(x)))))
            assert abs(Fraction(float(g)) - e) <= bd, (K, alpha, float(x))
    bd = np.asarray(bound(7, 1.5, 0.0, np.array([2.0, 3.0]), np.array([np.nan, np.inf])))
    assert np.all(np.isfinite(bd)) and np.all(bd > 0)


def _canary(K):
    """A = 1 + 2**-11 - 2**-23 (exact in FP32), B = 1, alpha = 1, beta = 0.
    Rounded to a 10-bit mantissa (binary16 / TF32 input precision) every
    a_k becomes 1, so such a path returns exactly K."""
    a = np.full((1, K), F32(1 + 2.0 ** -11 - 2.0 ** -23), F32)
    b = np.ones((K, 1), F32)
    return a, b


def round_mantissa(x, bits):
    """Round FP32 values to ``bits`` explicit mantissa bits, nearest-even."""
    m, e = np.frexp(np.asarray(x, np.float64))  # x = m * 2**e, 0.5 <= |m| < 1
    q = np.round(m * 2.0 ** (bits + 1)) / 2.0 ** (bits + 1)  # numpy rounds half to even
    return (q * 2.0 ** e).astype(F32)


def pin_bound_rejects_reduced_precision(bound):
    """Results from inputs held at a 10-bit (and a 7-bit) mantissa fail the
    bound at K = 1, 4, 64 and 1536, where it still sees that loss: error
    K*(2**-11 - 2**-23) against 4*K*2**-24*t with t ~ K, a ratio of about
    2047/K.  A bound looser by a factor of two (admits the K = 1536 case) or
    growing as K*K (admits K = 64) fails this pin."""
    for K in (1, 4, 64, 1536):
        a, b = _canary(K)
        for bits in (10, 7):
            ar = round_mantissa(a, bits)
            assert np.all(ar == 1.0)
            got = float(np.sum(ar.astype(np.float64)))  # = K, exact
            r, t, margin = _exact(a[0], b[:, 0], 1.0, 0.0, 0.0)
            bd = float(np.asarray(bound(K, 1.0, 0.0, np.float64(t), np.float64(np.nan))))
            assert abs(got - r) - margin > bd, (K, bits, abs(got - r), bd)
    # the R7 canary of the parity tests: A = 1 + m*2**-23 with low bits set,
    # B = 1, K <= 4; rounding A to 10 bits must be caught for every m tried
    rng = np.random.default_rng(43)
    for K in (1, 2, 3, 4):
        for _ in range(20):
            m = rng.integers(1, 2 ** 12, K) | 1
            a = F32(1 + m.astype(np.float64) * 2.0 ** -23)[None, :]
            b = np.ones((K, 1), F32)
            got = float(np.sum(round_mantissa(a, 10).astype(np.float64)))
            r, t, margin = _exact(a[0], b[:, 0], 1.0, 0.0, 0.0)
            bd = float(np.asarray(bound(K, 1.0, 0.0, np.float64(t), np.float64(0.0))))
            assert abs(got - r) - margin > bd, (K, m, abs(got - r), bd)


def pin_bound_golden(bound):
    """Values worked out by hand (tests/golden/error_bound.json)."""
    with open(GOLDEN, encoding="utf-8") as f:
        entries = json.load(f)["entries"]
    assert len(entries) >= 5
    for e in entries:
        c = float(e["c"]) if not isinstance(e["c"], str) else float(e["c"])
        got = float(np.asarray(bound(e["K"], e["alpha"], e["beta"], np.float64(e["t"]),
                                     np.float64(c))))
        want = e["bound_num"] / e["bound_den"]
        assert abs(got - want) <= 1e-15 * want, (e["id"], got, want)


ALL_BOUND_PINS = [
    pin_bound_admits_fp32_orders,
    pin_bound_admits_adversarial_sums,
    pin_bound_admits_k1_update,
    pin_bound_beta_and_empty_k,
    pin_bound_rejects_reduced_precision,
    pin_bound_golden,
]
