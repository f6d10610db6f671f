"""Reference SGEMM oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library under
``fp32_gemm_major_amd/`` and its binding) never imports it, and the two share
no code.

This module is argument marshalling around ``sgemm_oracle.c`` (plain C, FP64
accumulation, compiled with gcc -O2 and no fast-math).  What it computes is
the definition of the operation on the page "GEMM 优化之路", section on the
problem statement and performance limit: ``C = alpha*A*B + beta*C`` with
row-major FP32 operands, A M x K, B K x N, C M x N.  See the C source for the
exact arithmetic.  Results come back unrounded (FP64) as ``r``; the FP32
result of the operation is ``r`` rounded to nearest-even (``to_f32``).

``gemm_lowp`` is the same product with A and B stored as 16-bit patterns
(bfloat16 or IEEE binary16, ``DT_BF16`` / ``DT_F16``) or 8-bit patterns (the
OCP E4M3 and E5M2 formats, ``DT_FP8_E4M3`` / ``DT_FP8_E5M2``), C and the sums
as above: the mixed-precision matrix-unit product of the gsyq.cn guide,
section 5.1.

Pins (tests/test_oracle_pins.py) tie it to exact rational brute force, integer
arithmetic, identity and permutation matrices, the rank-1 closed form and the
alpha/beta semantics, none of which share code with it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "sgemm_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

# gcc flags: plain -O2, IEEE semantics (no -ffast-math, no FMA contraction
# of the additions is possible since every product is exact in FP64).
CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-pthread", "-fno-fast-math"]

_lock = threading.Lock()
_lib = None


def compile_library(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile ``source`` with gcc into the shared library ``output``."""
    tmp = output + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, "-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, output)
    return output


def build(force: bool = True) -> str:
    """Compile the oracle in place (always, unless ``force`` is False and it exists)."""
    global _lib
    with _lock:
        if force or not os.path.exists(LIBRARY):
            compile_library()
        _lib = None
    return LIBRARY


def _bind(lib):
    f = ctypes.c_float
    i = ctypes.c_int
    p = ctypes.c_void_p
    lib.oracle_sgemm_ex.argtypes = [i, i, i, i, i, f, p, i, p, i, f, p, i, p, i,
                                    p, i, i]
    lib.oracle_sgemm_ex.restype = i
    lib.oracle_sgemm_points_ex.argtypes = [i, i, i, i, i, f, p, i, p, i, f, p, i,
                                           i, p, p, p, p, i]
    lib.oracle_sgemm_points_ex.restype = i
    lib.oracle_gemm_lowp.argtypes = [i, i, i, i, i, i, f, p, i, p, i, f, p, i, p, i,
                                     p, i, i]
    lib.oracle_gemm_lowp.restype = i
    lib.oracle_gemm_lowp_points.argtypes = [i, i, i, i, i, i, f, p, i, p, i, f, p, i,
                                            i, p, p, p, p, i]
    lib.oracle_gemm_lowp_points.restype = i
    lib.oracle_gemm_fp8.argtypes = lib.oracle_gemm_lowp.argtypes
    lib.oracle_gemm_fp8.restype = i
    lib.oracle_gemm_fp8_points.argtypes = lib.oracle_gemm_lowp_points.argtypes
    lib.oracle_gemm_fp8_points.restype = i
    return lib


def load(path: str | None = None):
    """Load the compiled oracle (building it first only if it is missing)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(LIBRARY):
                compile_library()
            _lib = _bind(ctypes.CDLL(LIBRARY))
        return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f32(x, name):
    a = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    return a


def _ptr(a):
    return a.ctypes.data if a is not None and a.size else None


def _need(buf, rows, ld, cols, name):
    """Size a flat operand must have to hold ``rows`` rows of ``cols`` at stride ``ld``."""
    need = 0 if rows == 0 or cols == 0 else (rows - 1) * ld + cols
    if buf.size < need:
        raise ValueError(f"{name}: {buf.size} elements, need {need}")


def _need_ops(A, B, M, N, K, lda, ldb, ta, tb):
    if ta:
        _need(A, K, lda, M, "A (stored K x M)")
    else:
        _need(A, M, lda, K, "A")
    if tb:
        _need(B, N, ldb, K, "B (stored N x K)")
    else:
        _need(B, K, ldb, N, "B")


def gemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, *, with_t=True,
         nthreads=None, lib=None, ta=False, tb=False):
    """Full product.  Returns ``(r, t)``: FP64 arrays of shape (M, N).

    ``A``, ``B``, ``C`` are flat (or any-shape contiguous) FP32 buffers read at
    the given leading dimensions; ``C`` may be None when ``beta == 0``.
    ``t`` is None when ``with_t`` is False.  ``ta`` / ``tb``: A is stored
    K x M (A(i,k) = A[k*lda + i]) / B is stored N x K (B(k,j) = B[j*ldb + k]).
    """
    lib = lib or load()
    A = _f32(A, "A")
    B = _f32(B, "B")
    _need_ops(A, B, M, N, K, lda, ldb, ta, tb)
    if C is not None:
        C = _f32(C, "C")
        if beta != 0:
            _need(C, M, ldc, N, "C")
    elif beta != 0:
        raise ValueError("C is required when beta != 0")
    R = np.zeros((M, N), dtype=np.float64)
    T = np.zeros((M, N), dtype=np.float64) if with_t else None
    rc = lib.oracle_sgemm_ex(int(bool(ta)), int(bool(tb)), M, N, K, float(alpha),
                             _ptr(A), lda, _ptr(B), ldb, float(beta), _ptr(C), ldc,
                             _ptr(R), max(N, 1), _ptr(T), max(N, 1),
                             nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_sgemm rejected the arguments (code {rc})")
    return R, T


def gemm_points(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, rows, cols, *,
                nthreads=None, lib=None, ta=False, tb=False):
    """Outputs at (rows[p], cols[p]) only.  Returns ``(r, t)`` FP64 vectors."""
    lib = lib or load()
    A = _f32(A, "A")
    B = _f32(B, "B")
    _need_ops(A, B, M, N, K, lda, ldb, ta, tb)
    if C is not None:
        C = _f32(C, "C")
    elif beta != 0:
        raise ValueError("C is required when beta != 0")
    rows = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1)
    cols = np.ascontiguousarray(cols, dtype=np.int32).reshape(-1)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in length")
    n = rows.size
    r = np.zeros(n, dtype=np.float64)
    t = np.zeros(n, dtype=np.float64)
    rc = lib.oracle_sgemm_points_ex(int(bool(ta)), int(bool(tb)), M, N, K,
                                    float(alpha), _ptr(A), lda, _ptr(B), ldb,
                                    float(beta), _ptr(C), ldc, n, _ptr(rows),
                                    _ptr(cols), _ptr(r), _ptr(t),
                                    nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_sgemm_points rejected the arguments (code {rc})")
    return r, t


DT_BF16 = 1
DT_F16 = 2
DT_FP8_E4M3 = 3
DT_FP8_E5M2 = 4
_DT_NAMES = {"bf16": DT_BF16, "f16": DT_F16, "fp8e4m3": DT_FP8_E4M3,
             "fp8e5m2": DT_FP8_E5M2, DT_BF16: DT_BF16, DT_F16: DT_F16,
             DT_FP8_E4M3: DT_FP8_E4M3, DT_FP8_E5M2: DT_FP8_E5M2}


def _dt(dt):
    try:
        return _DT_NAMES[dt]
    except (KeyError, TypeError):
        raise ValueError(f"unknown 16-bit format {dt!r}") from None


def _bits(x, name, dt):
    """Flat bit-pattern array: uint16 for the 16-bit formats, uint8 for the
    8-bit ones."""
    want = np.uint8 if dt >= DT_FP8_E4M3 else np.uint16
    a = np.ascontiguousarray(x).reshape(-1)
    if a.dtype != want:
        raise ValueError(f"{name}: {np.dtype(want).name} bit patterns expected, got {a.dtype}")
    return a


def gemm_lowp(dt, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, *, with_t=True,
              nthreads=None, lib=None, ta=False, tb=False):
    """Full product with A and B stored as 16-bit patterns (uint16 arrays) or
    8-bit patterns (uint8 arrays).

    ``dt``: "bf16" / DT_BF16, "f16" / DT_F16, "fp8e4m3" / DT_FP8_E4M3 or
    "fp8e5m2" / DT_FP8_E5M2.  Everything else as ``gemm``.
    """
    dt = _dt(dt)
    lib = lib or load()
    A = _bits(A, "A", dt)
    B = _bits(B, "B", dt)
    _need_ops(A, B, M, N, K, lda, ldb, ta, tb)
    if C is not None:
        C = _f32(C, "C")
        if beta != 0:
            _need(C, M, ldc, N, "C")
    elif beta != 0:
        raise ValueError("C is required when beta != 0")
    R = np.zeros((M, N), dtype=np.float64)
    T = np.zeros((M, N), dtype=np.float64) if with_t else None
    fn = lib.oracle_gemm_fp8 if dt >= DT_FP8_E4M3 else lib.oracle_gemm_lowp
    rc = fn(dt, int(bool(ta)), int(bool(tb)), M, N, K, float(alpha),
                              _ptr(A), lda, _ptr(B), ldb, float(beta), _ptr(C), ldc,
                              _ptr(R), max(N, 1), _ptr(T), max(N, 1),
                              nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_gemm_lowp rejected the arguments (code {rc})")
    return R, T


def gemm_lowp_points(dt, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, rows, cols, *,
                     nthreads=None, lib=None, ta=False, tb=False):
    """Outputs of the 16-bit or 8-bit product at (rows[p], cols[p]) only."""
    dt = _dt(dt)
    lib = lib or load()
    A = _bits(A, "A", dt)
    B = _bits(B, "B", dt)
    _need_ops(A, B, M, N, K, lda, ldb, ta, tb)
    if C is not None:
        C = _f32(C, "C")
    elif beta != 0:
        raise ValueError("C is required when beta != 0")
    rows = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1)
    cols = np.ascontiguousarray(cols, dtype=np.int32).reshape(-1)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in length")
    n = rows.size
    r = np.zeros(n, dtype=np.float64)
    t = np.zeros(n, dtype=np.float64)
    fn = lib.oracle_gemm_fp8_points if dt >= DT_FP8_E4M3 else lib.oracle_gemm_lowp_points
    rc = fn(dt, int(bool(ta)), int(bool(tb)), M, N, K,
                                     float(alpha), _ptr(A), lda, _ptr(B), ldb,
                                     float(beta), _ptr(C), ldc, n, _ptr(rows),
                                     _ptr(cols), _ptr(r), _ptr(t),
                                     nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_gemm_lowp_points rejected the arguments (code {rc})")
    return r, t


def to_f32(r):
    """Round FP64 results to FP32, nearest-even (the oracle's FP32 output)."""
    return np.asarray(r, dtype=np.float64).astype(np.float32)


def error_bound(K, alpha, beta, t, c_in):
    """Per-element acceptance bound for an FP32 result against unrounded r.

    |C_gpu - r| <= 4 * max(K, 1) * 2**-24 * (|alpha| * t + |beta * c|), with the
    beta term taken as 0 when beta == 0 (C is then not read and may hold NaN).
    The form is the standard a-priori bound for a length-K FP32 dot product
    (gamma_K = K*u/(1 - K*u), u = 2**-24) widened to cover the few roundings of
    the alpha/beta update.  It holds unchanged for bfloat16 or binary16 A and B
    accumulated in FP32: the product of two such values is exact in FP32, so
    again only the FP32 additions round.  It does NOT cover products with 8-bit
    (E4M3 / E5M2) A and B on the matrix unit, whose instruction sums blocks of
    64 products in a narrower fixed-point window first: their tests add a
    per-block allowance to this bound (an envelope measured on the device, not
    a derived bound) and rely on integer inputs for exactness.  Pinned against
    FP32 arithmetic and hand-worked values in tests/bound_pins.py.
    """
    t = np.asarray(t, dtype=np.float64)
    scale = abs(float(alpha)) * t
    if beta != 0:
        scale = scale + np.abs(float(beta) * np.asarray(c_in, dtype=np.float64))
    return 4.0 * max(int(K), 1) * 2.0 ** -24 * scale
