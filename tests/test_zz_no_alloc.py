"""sgemm_run_ex_noalloc: the library's fixed scratch buffer in place of the
handle's workspace.  Its output must equal sgemm_run_ex's (same plan, same
deterministic kernels) and pass the oracle's acceptance, on two calls in a
row that both use the scratch buffer, the second on a smaller problem (so it
runs over what the first left behind)."""
import numpy as np
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
    # a workspace of exactly the fixed buffer's size: sgemm_run_ex then plans
    # what sgemm_run_ex_noalloc plans
    h = sg.Handle(workspace=False)
    h.set_workspace(sg.SGEMM_SCRATCH_BYTES)
    yield h
    h.close()


def _call(entry, h, ops, dev):
    A, B, C = dev
    entry(h.h, int(ops.ta), int(ops.tb), ops.M, ops.N, ops.K, ops.alpha, A.data_ptr(),
          ops.lda, B.data_ptr(), ops.ldb, ops.beta, C.data_ptr(), ops.ldc,
          torch.cuda.current_stream().cuda_stream)


# stream-K over 64x64 tiles (partial tiles in the buffer), then a smaller
# small-M problem whose K ranges keep their partial sums there
CASES = [(wl.Workload("na_sk", 9100, 64, 4096, 4096, 1.5, 0.5, "uniform"),
          sg.SGEMM_SCHEDULE_STREAM_K),
         (wl.Workload("na_small", 9101, 3, 2048, 8192, 1.0, 1.0, "int4"),
          sg.SGEMM_SCHEDULE_SMALL_M)]


def test_noalloc_matches_run_ex_twice_in_a_row(handle):
    prepared = []
    for w, schedule in CASES:
        ops = wl.operands(w)
        dev = gu.to_device(ops)
        plan = handle.plan(w.M, w.N, w.K, dev[0].data_ptr(), ops.lda, dev[1].data_ptr(),
                           ops.ldb, dev[2].data_ptr(), ops.ldc)
        assert [sg.sgemm_kernel_schedule(k) for k, _, _ in plan] == [schedule], plan
        if schedule == sg.SGEMM_SCHEDULE_SMALL_M:  # a kernel that splits K, not a one-pass one
            name = sg.sgemm_kernel_name(plan[0][0])
            assert "splitk" in name or "x256" in name, name
        c0 = dev[2].clone()
        _call(sg.sgemm_run_ex, handle, ops, dev)
        torch.cuda.synchronize()
        ref = dev[2].cpu().numpy().copy()
        dev[2].copy_(c0)
        prepared.append((w, ops, dev, ref))
    torch.cuda.synchronize()
    # the two calls back to back, the second smaller
    for w, ops, dev, _ in prepared:
        _call(sg.sgemm_run_ex_noalloc, handle, ops, dev)
    torch.cuda.synchronize()
    for w, ops, dev, ref in prepared:
        out = dev[2].cpu().numpy()
        assert np.array_equal(out.view(np.uint32), ref.view(np.uint32)), w.name
        gu.check_full(ops, out, exact=w.dist == "int4", what=f"noalloc {w.name}")


def test_noalloc_refuses_a_forced_kernel_beyond_the_buffer(handle):
    """A forced stream-K kernel whose partial tiles need more than the fixed
    buffer (128x128: 64 MiB on 256 CUs) is refused before any launch."""
    k = next(k for k in sg.kernel_table() if k["schedule"] == sg.SGEMM_SCHEDULE_STREAM_K
             and k["bm"] == 128 and k["mode"] == sg.SGEMM_MODE_ALIGNED
             and not k["transa"] and not k["transb"])
    w = wl.Workload("na_big", 9102, 512, 512, 4096, 1.0, 1.0, "int4")
    ops = wl.operands(w)
    dev = gu.to_device(ops)
    c0 = dev[2].clone()
    handle.set_kernel(k["id"])
    try:
        with pytest.raises(sg.SgemmError) as e:
            _call(sg.sgemm_run_ex_noalloc, handle, ops, dev)
        assert e.value.status == sg.SGEMM_ERR_SCRATCH
    finally:
        handle.set_kernel(-1)
    torch.cuda.synchronize()
    assert torch.equal(dev[2], c0)


def test_noalloc_argument_errors_and_empty_problems(handle):
    A = torch.ones(64 * 64, device="cuda")
    B = torch.ones(64 * 64, device="cuda")
    with pytest.raises(sg.SgemmError) as e:
        sg.sgemm_run_ex_noalloc(handle.h, 0, 0, 64, 64, 64, 1.0, A.data_ptr(), 64,
                                B.data_ptr(), 64, 0.0, A.data_ptr(), 64)
    assert e.value.status == sg.SGEMM_ERR_ALIAS
    C = torch.full((64 * 64,), 2.0, device="cuda")
    assert sg.sgemm_run_ex_noalloc(handle.h, 0, 0, 0, 64, 64, 1.0, A.data_ptr(), 64,
                                   B.data_ptr(), 64, 0.0, C.data_ptr(), 64) == 0
    torch.cuda.synchronize()
    assert torch.all(C == 2.0)
