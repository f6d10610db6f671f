"""Calls captured in a HIP graph and replayed.

Every kind of launch plan -- one tile per workgroup, two launches over column
ranges, stream-K with its fixup, split K with its reduction, the one-pass
small-M kernel, the fixed-scratch entry point, and the 16/8-bit tile, split-K
and one-pass kernels -- is
captured once, then replayed three times with the program's own eager work
between the replays (C restored from a copy, an unrelated product, host
synchronisations).  Every replay must give the eager call's bits: the
kernels are deterministic and record no memset, so a replay can differ only
through state a kernel leaves behind.  Each case also passes the oracle.
"""
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import fp32_gemm_major_amd as sg  # noqa: E402
from fp32_gemm_major_amd import workloads as wl  # noqa: E402
from tests import gpu_util as gu  # noqa: E402


@pytest.fixture(scope="module")
def handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h = sg.Handle()  # with a workspace: stream-K and split-K plans can run
    yield h
    h.close()


def _replays_match(call, C, c0, what):
    """Eager call, then three replays of a captured one, each against it."""
    C.copy_(c0)
    call()
    torch.cuda.synchronize()
    ref = C.clone()
    g = torch.cuda.CUDAGraph()
    C.copy_(c0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call()
    x = torch.rand(512, 512, device="cuda")
    for r in range(3):
        C.copy_(c0)                      # eager work between the replays
        y = x @ x
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C.view(torch.int32), ref.view(torch.int32)), (what, r)
        assert torch.isfinite(y).all()
    del g
    return ref


def _fp32_kernel_schedule(h, ops, dev):
    A, B, C = dev
    plan = h.plan(ops.M, ops.N, ops.K, A.data_ptr(), ops.lda, B.data_ptr(), ops.ldb,
                  C.data_ptr(), ops.ldc, transa=ops.ta, transb=ops.tb)
    return [sg.sgemm_kernel_schedule(k) for k, _, _ in plan]


# (workload, storage flags, the schedules of the launches its plan must make:
# 2048 x 5504 x 2048 is two launches, whole rounds of 128x128 tiles over the
# first 4096 columns and 64x64 tiles over the rest)
FP32_CASES = [
    (wl.Workload("g_tiles", 9200, 512, 384, 256, 1.5, 0.5, "uniform"), (False, False),
     [sg.SGEMM_SCHEDULE_TILES]),
    (wl.Workload("g_edge", 9201, 1000, 1500, 777, 1.0, 1.0, "uniform"), (False, False), None),
    (wl.Workload("g_sk", 9202, 64, 4096, 4096, 1.5, 0.5, "uniform"), (False, False),
     [sg.SGEMM_SCHEDULE_STREAM_K]),
    (wl.Workload("g_splitk", 9203, 16, 4096, 4096, 1.0, 0.5, "uniform"), (False, True),
     [sg.SGEMM_SCHEDULE_SMALL_M]),
    (wl.Workload("g_onepass", 9206, 4, 4096, 4096, 1.0, 0.5, "uniform"), (False, True),
     [sg.SGEMM_SCHEDULE_SMALL_M]),
    (wl.Workload("g_onepass_kn", 9207, 1, 4096, 4096, 1.0, 0.5, "uniform"), (False, False),
     [sg.SGEMM_SCHEDULE_SMALL_M]),
    (wl.Workload("g_two", 9204, 2048, 5504, 2048, 1.0, 0.0, "normal"), (False, False),
     [sg.SGEMM_SCHEDULE_TILES, sg.SGEMM_SCHEDULE_TILES]),
]


@pytest.mark.parametrize("case", FP32_CASES, ids=[c[0].name for c in FP32_CASES])
def test_fp32_plans_replay(handle, case):
    w, (ta, tb), want = case
    ops = wl.operands(w, ta=ta, tb=tb)
    dev = gu.to_device(ops)
    sched = _fp32_kernel_schedule(handle, ops, dev)
    if want is not None:
        assert sched == want, sched
    A, B, C = dev
    c0 = C.clone()

    def call():
        handle.gemm(A, B, C, ops.alpha, ops.beta, M=ops.M, N=ops.N, K=ops.K, lda=ops.lda,
                    ldb=ops.ldb, ldc=ops.ldc, transa=ta, transb=tb)
    _replays_match(call, C, c0, w.name)
    out = C.cpu().numpy()[: ops.C.size].copy()
    if w.M * w.N * w.K <= 2 ** 31:
        gu.check_full(ops, out, what=f"{w.name} replayed")
    else:
        gu.check_sampled(ops, out, [0, w.M - 1], [0, w.N - 1], what=f"{w.name} replayed")


def test_noalloc_replay(handle):
    """The fixed-scratch entry point under capture: a stream-K plan whose
    partial tiles live in the library's buffer."""
    w = wl.Workload("g_na", 9205, 64, 4096, 4096, 1.5, 0.5, "uniform")
    ops = wl.operands(w)
    A, B, C = gu.to_device(ops)
    c0 = C.clone()

    def call():
        sg.sgemm_run_ex_noalloc(handle.h, 0, 0, ops.M, ops.N, ops.K, ops.alpha,
                                A.data_ptr(), ops.lda, B.data_ptr(), ops.ldb, ops.beta,
                                C.data_ptr(), ops.ldc, torch.cuda.current_stream().cuda_stream)
    _replays_match(call, C, c0, w.name)
    gu.check_full(ops, C.cpu().numpy()[: ops.C.size].copy(), what="noalloc replayed")


LOWP_CASES = [
    ("bf16", wl.Workload("g_lp", 9210, 512, 512, 512, 1.5, 0.5, "uniform"), False),
    ("fp8e4m3", wl.Workload("g_lp8", 9211, 300, 260, 777, 1.0, 1.0, "int4"), True),
    ("bf16", wl.Workload("g_lpsk", 9212, 1, 4096, 4096, 1.0, 0.5, "uniform"), False),
    ("fp8e4m3", wl.Workload("g_gemv", 9213, 3, 4096, 4096, 1.0, 0.5, "int4"), True),
    ("f16", wl.Workload("g_gemv16", 9214, 1, 4096, 4096, 1.0, 0.0, "uniform"), True),
]


@pytest.mark.parametrize("case", LOWP_CASES, ids=[c[1].name for c in LOWP_CASES])
def test_lowp_plans_replay(handle, case):
    dt, w, tb = case
    ops = wl.operands16(w, dt, tb=tb)
    A, B, C = gu.to_device16(ops)
    c0 = C.clone()

    def call():
        handle.gemm_lowp(A, B, C, ops.alpha, ops.beta, M=ops.M, N=ops.N, K=ops.K,
                         lda=ops.lda, ldb=ops.ldb, ldc=ops.ldc, transb=tb)
    _replays_match(call, C, c0, w.name)
    gu.check_full16(ops, C.cpu().numpy()[: ops.C.size].copy(), exact=w.dist == "int4",
                    what=f"{w.name} replayed")
