"""Work and traffic accounting for one SGEMM, and MI355X peak figures.

The counts follow "GEMM 优化之路" (problem statement and performance limit):
an M x N x K product does 2*M*N*K floating-point operations (one multiply and
one add per term; the alpha/beta update is not counted, as on the page), and
the least traffic is one read of A and B plus the C traffic: a read and a
write of C when beta != 0, a write only when beta == 0 (the page gives both
totals, ~268 MB and ~200 MB, for 4096^3).  Exercise 1 on the same page counts
the operand loads of a tiled kernel as 2 * tile * K * 4 bytes per square
block; ``tile_loads`` is the general rectangular form.
"""
from __future__ import annotations

FP32 = 4  # bytes

# MI355X published peaks: 256 CUs x 2.4 GHz x 256 FP32 FLOP/clk/CU (FP32
# matrix cores; packed FP32 vector FMA has the same peak), and HBM3E.
PEAK_FP32_FLOPS = 157.3e12
PEAK_FP32_VALU_UNPACKED_FLOPS = PEAK_FP32_FLOPS / 2  # one FMA per lane per clock
# Dense (no sparsity) matrix-core peaks for 16-bit inputs with FP32
# accumulation: bfloat16 and binary16 alike.
PEAK_BF16_FLOPS = 2.5e15
PEAK_F16_FLOPS = 2.5e15
# ... and for 8-bit (OCP E4M3 / E5M2) inputs.
PEAK_FP8_FLOPS = 5.0e15
PEAK_HBM_BYTES = 8.0e12
CUS = 256
CLOCK_HZ = 2.4e9
FP32_FLOPS_PER_CU_CLOCK = 256  # 157.3e12 = 256 CUs x 2.4e9 x 256


def flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def alg_bytes(M: int, N: int, K: int, beta: float, ab_bytes: int = FP32) -> int:
    """Least HBM traffic: A and B read once (``ab_bytes`` per element: 2 for
    16-bit operands, 1 for 8-bit ones), FP32 C written (and read if
    beta != 0)."""
    c_passes = 2 if beta != 0 else 1
    return ab_bytes * (M * K + K * N) + FP32 * c_passes * M * N


def arithmetic_intensity(M: int, N: int, K: int, beta: float) -> float:
    return flops(M, N, K) / alg_bytes(M, N, K, beta)


def ridge_point(peak_flops: float, peak_bytes: float) -> float:
    return peak_flops / peak_bytes


def tiles(M: int, N: int, BM: int, BN: int) -> int:
    return -(-M // BM) * -(-N // BN)


def tile_loads(M: int, N: int, K: int, BM: int, BN: int) -> int:
    """Operand bytes all blocks of a BM x BN tiling load (before any cache)."""
    return tiles(M, N, BM, BN) * (BM + BN) * K * FP32


def seconds_at_peak(M: int, N: int, K: int, peak=PEAK_FP32_FLOPS) -> float:
    return flops(M, N, K) / peak
