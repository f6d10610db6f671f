"""The acceptance of the 8-bit kernels (the FP32 bound plus the per-block
allowance of the 8-bit matrix instruction, tests/gpu_util.py) still catches
the mistakes parity is there to catch: a result that misses one product per
output, or takes one from the wrong k, fails it for most outputs.  CPU only:
the "results" are the oracle's own, changed on the CPU."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from fp32_gemm_major_amd import workloads as wl  # noqa: E402
from tests import gpu_util as gu  # noqa: E402


def _decoded(bits, dt, rows, ld, cols):
    x = torch.from_numpy(bits[: rows * ld].reshape(rows, ld)[:, :cols].copy())
    return x.view(gu.TORCH_FORMATS[dt]).to(torch.float64).numpy()


@pytest.mark.parametrize("dt", wl.FORMATS8)
@pytest.mark.parametrize("name", ["c1_128", "c4_edge"])
def test_allowance_catches_a_dropped_or_misindexed_product(dt, name):
    w = wl.WORKLOADS[name]
    if name == "c4_edge":
        w = wl.Workload(w.name, w.cfg_id, 96, 80, w.K, w.alpha, w.beta, w.dist)
    ops = wl.operands16(w, dt, tb=True)
    M, N, K = ops.M, ops.N, ops.K
    R, T = oracle.gemm_lowp(dt, M, N, K, ops.alpha, ops.A, ops.lda, ops.B, ops.ldb,
                            ops.beta, ops.C, ops.ldc, tb=True)
    a = _decoded(ops.A, dt, M, ops.lda, K)
    b = _decoded(ops.B, dt, N, ops.ldb, K)
    c_in = gu.window(ops.C, M, N, ops.ldc)
    extra = gu.fp8_extra(ops, np.arange(M)[:, None], np.arange(N)[None, :])
    bound = oracle.error_bound(K, ops.alpha, ops.beta, T, c_in) + extra
    # the oracle's own result passes
    gu.check(oracle.to_f32(R), R, T, K, ops.alpha, ops.beta, c_in, what="oracle", extra=extra)
    k = K // 2
    dropped = ops.alpha * a[:, k][:, None] * b[:, k][None, :]
    shifted = ops.alpha * (a[:, k + 1][:, None] - a[:, k][:, None]) * b[:, k][None, :]
    for change, what in ((dropped, "dropped"), (shifted, "k+1 in place of k")):
        wrong = oracle.to_f32(R - change)
        caught = np.abs(wrong.astype(np.float64) - R) > bound
        assert caught.mean() > 0.75, (what, caught.mean())
        with pytest.raises(AssertionError):
            gu.check(wrong, R, T, K, ops.alpha, ops.beta, c_in, what=what, extra=extra)
