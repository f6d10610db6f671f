"""Seeded synthetic workloads for the SGEMM path.

This module only names problem sizes and draws inputs.  It holds none of the
operation's arithmetic, so both sides of every parity check (the HIP library
and the CPU oracle used by the tests) can take their inputs from it.

Shapes and value distributions follow the pages' workloads:
* square sizes 128, 1024 and 4096 and the headline 4096^3 problem
  ("GEMM 优化之路", problem statement and its complete listing's main program,
  which checks at n = 512 with alpha = 1, beta = 0.5 and times at 4096);
* a size that is not a tile multiple, 1000 x 1500 x 777 (same page, exercise 2,
  which asks for 1000 x 999 x 777);
* the transformer MLP up-projection shape 4096 x 11008 x 4096.

Uniform values are ``2*U - 1`` with U an FP32 uniform on [0, 1) from numpy's
PCG64, giving exactly representable values in [-1, 1 - 2**-23].  The T4 page's
generator draws ``rand()/RAND_MAX*2 - 1`` on the closed interval; the half-open
FP32 grid is the plain reading that keeps every value exact in FP32.
Integer variants draw from {-4, ..., 4}; every partial sum of such inputs at
these sizes is an integer below 2**24, so any summation order is exact.
Every operand is drawn from ``default_rng([cfg_id, role])`` with role A=1,
B=2, C=3, so values do not depend on the leading dimensions chosen.

Products with 16-bit A and B (bfloat16 or IEEE binary16, FP32 C) draw the same
FP32 values and round them to the 16-bit format, nearest-even
(``round16``); the bit patterns are what both sides receive.  Products with
8-bit A and B (the OCP E4M3 and E5M2 formats) round them the same way with
torch's conversions (``round8``).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

ROLE_A, ROLE_B, ROLE_C = 1, 2, 3


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    M: int
    N: int
    K: int
    alpha: float
    beta: float
    dist: str  # "uniform" | "normal" | "int4"
    c_fill: str = "dist"  # "dist": drawn like A, B; "nan": never read (beta == 0)

    @property
    def label(self) -> str:
        return (f"sgemm_{self.M}x{self.N}x{self.K}_a{self.alpha:g}_b{self.beta:g}"
                f"_{self.dist}")


WORKLOADS = {
    "c1_128": Workload("c1_128", 1, 128, 128, 128, 1.0, 0.0, "uniform"),
    "c1_128_int": Workload("c1_128_int", 101, 128, 128, 128, 1.0, 0.0, "int4"),
    "c2_1024": Workload("c2_1024", 2, 1024, 1024, 1024, 1.0, 0.0, "uniform", "nan"),
    "c3_4096": Workload("c3_4096", 3, 4096, 4096, 4096, 1.5, 0.5, "uniform"),
    "c3_4096_int": Workload("c3_4096_int", 103, 4096, 4096, 4096, 1.5, 0.5, "int4"),
    "c4_edge": Workload("c4_edge", 4, 1000, 1500, 777, 1.0, 1.0, "uniform"),
    "c4_edge_int": Workload("c4_edge_int", 104, 1000, 1500, 777, 1.0, 1.0, "int4"),
    "c5_mlp": Workload("c5_mlp", 5, 4096, 11008, 4096, 1.0, 0.0, "normal", "nan"),
}

# The headline workload timed by the benchmark.
HEADLINE = "c3_4096"


def draw(cfg_id: int, role: int, rows: int, cols: int, dist: str) -> np.ndarray:
    """Dense (rows, cols) FP32 array of seeded values."""
    rng = np.random.default_rng([cfg_id, role])
    shape = (rows, cols)
    if dist == "uniform":
        return 2.0 * rng.random(shape, dtype=np.float32) - np.float32(1.0)
    if dist == "normal":
        return rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)
    if dist == "int4":
        return rng.integers(-4, 5, size=shape).astype(np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


FORMATS16 = ("bf16", "f16")


def round16(values: np.ndarray, dt: str) -> np.ndarray:
    """Bit patterns (uint16) of FP32 ``values`` rounded to the nearest bfloat16
    or IEEE binary16 value, ties to even (inputs must be finite).

    binary16 is numpy's own conversion.  bfloat16 keeps the upper half of the
    binary32 pattern after adding half an ulp of the kept part (0x7FFF plus the
    kept part's lowest bit, which sends ties to the even neighbour).
    """
    x = np.ascontiguousarray(values, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("round16 takes finite values only")
    if dt == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dt == "bf16":
        w = x.view(np.uint32).astype(np.uint64)
        w = (w + 0x7FFF + ((w >> 16) & 1)) >> 16
        return w.astype(np.uint16)
    raise ValueError(f"unknown 16-bit format {dt!r}")


FORMATS8 = ("fp8e4m3", "fp8e5m2")


def round8(values: np.ndarray, dt: str) -> np.ndarray:
    """Bit patterns (uint8) of FP32 ``values`` rounded to the nearest E4M3 or
    E5M2 value, ties to even (torch's conversions; values must lie inside the
    format's finite range)."""
    import torch

    x = np.ascontiguousarray(values, dtype=np.float32)
    tdt = {"fp8e4m3": torch.float8_e4m3fn, "fp8e5m2": torch.float8_e5m2}.get(dt)
    if tdt is None:
        raise ValueError(f"unknown 8-bit format {dt!r}")
    limit = 448.0 if dt == "fp8e4m3" else 57344.0
    if not np.all(np.isfinite(x)) or np.abs(x).max(initial=0.0) > limit:
        raise ValueError("round8 takes values inside the format's finite range")
    return torch.from_numpy(x).to(tdt).view(torch.uint8).numpy().copy()


def place16(bits: np.ndarray, ld: int, pad_value=None) -> np.ndarray:
    """``place`` for 16-bit or 8-bit patterns; padding defaults to a NaN
    pattern of the formats of that width (0x7FC0 is a quiet NaN in bfloat16
    and binary16, 0x7F in E4M3 and E5M2)."""
    if pad_value is None:
        pad_value = 0x7F if bits.dtype == np.uint8 else 0x7FC0
    rows, cols = bits.shape
    if ld < cols:
        raise ValueError("ld < cols")
    buf = np.full((rows, ld), pad_value, dtype=bits.dtype)
    buf[:, :cols] = bits
    return buf.reshape(-1)


def place(values: np.ndarray, ld: int, pad_value=np.nan) -> np.ndarray:
    """Store a (rows, cols) array row-major at leading dimension ``ld``.

    Returns a flat FP32 buffer of rows*ld elements; the ``ld - cols`` padding
    entries of each row hold ``pad_value`` (NaN by default, so that a read of
    padding poisons the result and a write to it is visible).
    """
    rows, cols = values.shape
    if ld < cols:
        raise ValueError("ld < cols")
    buf = np.full((rows, ld), pad_value, dtype=np.float32)
    buf[:, :cols] = values
    return buf.reshape(-1)


@dataclass
class Operands:
    M: int
    N: int
    K: int
    alpha: float
    beta: float
    A: np.ndarray  # flat: M rows of lda (K rows of lda when ta)
    lda: int
    B: np.ndarray  # flat: K rows of ldb (N rows of ldb when tb)
    ldb: int
    C: np.ndarray  # flat, M*ldc (C_in)
    ldc: int
    ta: bool = False  # A stored transposed (K x M)
    tb: bool = False  # B stored transposed (N x K)


def operands(w: Workload, lda=None, ldb=None, ldc=None, pad_value=np.nan,
             M=None, N=None, K=None, ta=False, tb=False) -> Operands:
    """Inputs of workload ``w`` (optionally with other sizes or leading dims).

    ``ta`` / ``tb`` store A as its transpose (K x M) / B as its transpose
    (N x K); the logical values are the same as without them.
    """
    if M is not None or N is not None or K is not None:
        w = replace(w, M=w.M if M is None else M, N=w.N if N is None else N,
                    K=w.K if K is None else K)
    lda = max(w.M if ta else w.K, 1) if lda is None else lda
    ldb = max(w.K if tb else w.N, 1) if ldb is None else ldb
    ldc = max(w.N, 1) if ldc is None else ldc
    a = draw(w.cfg_id, ROLE_A, w.M, w.K, w.dist)
    b = draw(w.cfg_id, ROLE_B, w.K, w.N, w.dist)
    if ta:
        a = np.ascontiguousarray(a.T)
    if tb:
        b = np.ascontiguousarray(b.T)
    if w.c_fill == "nan":
        c = np.full((w.M, w.N), np.nan, dtype=np.float32)
    else:
        c = draw(w.cfg_id, ROLE_C, w.M, w.N, w.dist)
    return Operands(w.M, w.N, w.K, w.alpha, w.beta,
                    place(a, lda, pad_value), lda,
                    place(b, ldb, pad_value), ldb,
                    place(c, ldc, pad_value), ldc, ta, tb)


@dataclass
class Operands16:
    """Operands of the product with 16-bit or 8-bit A and B (bit patterns)
    and FP32 C."""
    dt: str
    M: int
    N: int
    K: int
    alpha: float
    beta: float
    A: np.ndarray  # flat uint16 / uint8: M rows of lda (K rows of lda when ta)
    lda: int
    B: np.ndarray  # flat uint16 / uint8: K rows of ldb (N rows of ldb when tb)
    ldb: int
    C: np.ndarray  # flat FP32, M*ldc (C_in)
    ldc: int
    ta: bool = False
    tb: bool = False


def operands16(w: Workload, dt: str, lda=None, ldb=None, ldc=None, M=None, N=None,
               K=None, ta=False, tb=False) -> Operands16:
    """Inputs of workload ``w`` with A and B rounded to the 16-bit or 8-bit
    format ``dt``; C is drawn exactly as in ``operands``."""
    if M is not None or N is not None or K is not None:
        w = replace(w, M=w.M if M is None else M, N=w.N if N is None else N,
                    K=w.K if K is None else K)
    lda = max(w.M if ta else w.K, 1) if lda is None else lda
    ldb = max(w.K if tb else w.N, 1) if ldb is None else ldb
    ldc = max(w.N, 1) if ldc is None else ldc
    rnd = round8 if dt in FORMATS8 else round16
    a = rnd(draw(w.cfg_id, ROLE_A, w.M, w.K, w.dist), dt)
    b = rnd(draw(w.cfg_id, ROLE_B, w.K, w.N, w.dist), dt)
    if ta:
        a = np.ascontiguousarray(a.T)
    if tb:
        b = np.ascontiguousarray(b.T)
    if w.c_fill == "nan":
        c = np.full((w.M, w.N), np.nan, dtype=np.float32)
    else:
        c = draw(w.cfg_id, ROLE_C, w.M, w.N, w.dist)
    return Operands16(dt, w.M, w.N, w.K, w.alpha, w.beta,
                      place16(a, lda), lda, place16(b, ldb), ldb,
                      place(c, ldc), ldc, ta, tb)
