"""Parity of the HIP SGEMM (through the C ABI) with the FP64 CPU oracle.

Acceptance, elementwise over the M x N window:
|C_gpu - r| <= 4*max(K,1)*2^-24*(|alpha|*sum_k|a_ik*b_kj| + |beta*c_ij|), with
r the unrounded FP64 result; bit-exact (== r rounded to FP32) for integer
inputs, whose partial sums are all exact in FP32.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import fp32_gemm_major_amd as sg  # noqa: E402
import oracle  # noqa: E402
from fp32_gemm_major_amd import workloads as wl  # noqa: E402
from tests import gpu_util as gu  # noqa: E402

W = wl.WORKLOADS


@pytest.fixture(scope="module")
def handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h = sg.Handle()
    yield h
    h.close()


@pytest.fixture(autouse=True)
def _auto_kernel(handle):
    handle.set_kernel(-1)
    handle.set_variant(sg.SGEMM_VARIANT_AUTO)
    yield
    handle.set_kernel(-1)
    handle.set_variant(sg.SGEMM_VARIANT_AUTO)


KERNELS = [] if not __import__("os").path.exists(sg.LIBRARY) else sg.kernel_table()


def edge_fit(k, M, N):
    """Raise M / N to what an edge instance takes: at least 4 along the
    operand whose 16-byte pieces run along M (A^T) or N (B as stored)."""
    if k["mode"] == sg.SGEMM_MODE_EDGE:
        if k["transa"]:
            M = max(M, 4)
        if not k["transb"]:
            N = max(N, 4)
    return M, N


# ---- every kernel of the table, on problems spanning several tiles ----------

@pytest.mark.parametrize("k", KERNELS, ids=[k["name"] for k in KERNELS])
@pytest.mark.parametrize("dist", ["uniform", "int4"])
def test_each_kernel(handle, k, dist):
    handle.set_kernel(k["id"])
    if k["schedule"] == sg.SGEMM_SCHEDULE_SMALL_M:  # at most bm rows
        M, N, K = k["bm"], 2 * k["bn"] + 19, 3 * k["bk"] + 5
        lda, ldb, ldc = K + 3, N + 1, N + 5
    elif k["mode"] != sg.SGEMM_MODE_ALIGNED:
        M, N = edge_fit(k, 2 * k["bm"] + 37, k["bn"] + 19)
        K = 3 * k["bk"] + 5
        lda, ldb, ldc = K + 3, N + 1, N + 5
    else:
        M, N, K = 2 * k["bm"], 3 * k["bn"], 4 * k["bk"]
        # MFMA direct loads take rows that are only 4-byte aligned
        pad = 1 if k["variant"] == sg.SGEMM_VARIANT_MFMA else 0
        lda, ldb, ldc = K + pad, N + 3 * pad, N + 4
    ta, tb = bool(k["transa"]), bool(k["transb"])
    if ta:  # stored K x M
        lda = M + (lda - K)
    if tb:  # stored N x K
        ldb = K + (ldb - N)
    w = wl.Workload("case", 900 + k["id"], M, N, K, 1.5, 0.5, dist)
    ops = wl.operands(w, lda=lda, ldb=ldb, ldc=ldc, ta=ta, tb=tb)
    out = gu.run(handle, ops)
    gu.check_full(ops, out, exact=(dist == "int4"), what=k["name"])


# ---- the five workloads, in the configuration the benchmark runs ------------

def test_c1_uniform(handle):
    ops = wl.operands(W["c1_128"])
    gu.check_full(ops, gu.run(handle, ops), what="c1")


def test_c1_integer_bit_exact(handle):
    ops = wl.operands(W["c1_128_int"])
    gu.check_full(ops, gu.run(handle, ops), exact=True, what="c1 int")


def test_c2_nan_c_beta_zero(handle):
    ops = wl.operands(W["c2_1024"])
    assert np.all(np.isnan(ops.C))
    gu.check_full(ops, gu.run(handle, ops), what="c2")


def test_c3_headline_full(handle):
    """Every output of the 4096^3 problem against the full oracle."""
    ops = wl.operands(W["c3_4096"])
    gu.check_full(ops, gu.run(handle, ops), what="c3")


def test_c3_integer_bit_exact(handle):
    ops = wl.operands(W["c3_4096_int"])
    gu.check_full(ops, gu.run(handle, ops), exact=True, what="c3 int")


def test_c4_edge_full(handle):
    ops = wl.operands(W["c4_edge"])
    gu.check_full(ops, gu.run(handle, ops), what="c4")


def test_c4_edge_integer_bit_exact(handle):
    ops = wl.operands(W["c4_edge_int"])
    gu.check_full(ops, gu.run(handle, ops), exact=True, what="c4 int")


def test_c5_mlp_full(handle):
    ops = wl.operands(W["c5_mlp"])
    gu.check_full(ops, gu.run(handle, ops), what="c5")


@pytest.mark.parametrize("name", ["c3_4096", "c4_edge"])
def test_valu_variant(handle, name):
    handle.set_variant(sg.SGEMM_VARIANT_VALU)
    w = W[name]
    ops = wl.operands(w)
    out = gu.run(handle, ops)
    if w.M * w.N * w.K > 2e9:
        gu.check_sampled(ops, out, gu.edge_rows(w.M, extra=2), cols=[0, 4095],
                         what=name + " valu")
    else:
        gu.check_full(ops, out, what=name + " valu")


# ---- transposed operands (op(A) = A^T, op(B) = B^T) ---------------------------

OPS = [(False, True), (True, False), (True, True)]


@pytest.mark.parametrize("ta,tb", OPS, ids=["nt", "tn", "tt"])
def test_transposed_aligned(handle, ta, tb):
    w = wl.Workload("trans", 6000, 1024, 1536, 768, 1.5, 0.5, "uniform")
    ops = wl.operands(w, ta=ta, tb=tb)
    gu.check_full(ops, gu.run(handle, ops), what=f"trans {ta}{tb}")


@pytest.mark.parametrize("ta,tb", OPS, ids=["nt", "tn", "tt"])
def test_transposed_edges_integer(handle, ta, tb):
    w = wl.Workload("trans", 6001, 1000, 1500, 777, 1.0, 1.0, "int4")
    ops = wl.operands(w, ta=ta, tb=tb)
    gu.check_full(ops, gu.run(handle, ops), exact=True, what=f"trans edge {ta}{tb}")


@pytest.mark.parametrize("ta,tb", OPS, ids=["nt", "tn", "tt"])
def test_transposed_4096_split_plan(handle, ta, tb):
    """4096 x 4352 x 512 runs as two column launches; op(B) = B^T offsets B by rows."""
    w = wl.Workload("trans", 6002, 4096, 4352, 512, 1.0, 0.0, "normal", "nan")
    ops = wl.operands(w, ta=ta, tb=tb)
    plan = sg.sgemm_plan(0, w.M, w.N, w.K, 0x10000000, ops.lda, 0x20000000, ops.ldb,
                         0x40000000, ops.ldc, transa=int(ta), transb=int(tb))
    assert len(plan) == 2
    gu.check_full(ops, gu.run(handle, ops), what=f"trans split {ta}{tb}")


def test_valu_has_no_transposes(handle):
    handle.set_variant(sg.SGEMM_VARIANT_VALU)
    A = torch.ones(64 * 64, device="cuda")
    B = torch.ones(64 * 64, device="cuda")
    C = torch.zeros(64 * 64, device="cuda")
    with pytest.raises(sg.SgemmError) as e:
        handle.gemm(A, B, C, 1.0, 0.0, M=64, N=64, K=64, lda=64, ldb=64, ldc=64,
                    transa=True)
    assert e.value.status == sg.SGEMM_ERR_UNSUPPORTED


def test_k_not_a_multiple_of_the_stage(handle):
    """K a multiple of 16 but not of 64: the 64x64 tile's stage holds 64 k, so
    its aligned instance must not be used (it would read past K)."""
    for K in (1040, 80, 16):
        w = wl.Workload("kstage", 6003, 256, 192, K, 1.0, 0.0, "int4", "nan")
        ops = wl.operands(w)
        gu.check_full(ops, gu.run(handle, ops), exact=True, what=f"K={K}")


# ---- edge cases -----------------------------------------------------------------

TINY = sorted({(m, n, k) for m in (1, 2, 31, 32, 33, 64, 65, 70)
               for n in (1, 3, 32, 63, 64, 70) for k in (1, 4, 15, 16, 17, 70)
               if (m * 7 + n * 3 + k) % 4 == 0} | {(1, 1, 1), (70, 70, 70), (5, 9, 0)})


@pytest.mark.parametrize("variant", [sg.SGEMM_VARIANT_MFMA, sg.SGEMM_VARIANT_VALU])
def test_tiny_sizes_integer_exact(handle, variant):
    handle.set_variant(variant)
    for i, (M, N, K) in enumerate(TINY):
        w = wl.Workload("tiny", 2000 + i, M, N, K, 1.0, -1.0, "int4")
        ops = wl.operands(w)
        gu.check_full(ops, gu.run(handle, ops), exact=True, what=f"tiny {M}x{N}x{K}")


@pytest.mark.parametrize("variant", [sg.SGEMM_VARIANT_MFMA, sg.SGEMM_VARIANT_VALU])
def test_tiny_sizes_uniform(handle, variant):
    handle.set_variant(variant)
    for i, (M, N, K) in enumerate(TINY[::3]):
        w = wl.Workload("tiny", 3000 + i, M, N, K, 1.5, 0.5, "uniform")
        ops = wl.operands(w)
        gu.check_full(ops, gu.run(handle, ops), what=f"tiny {M}x{N}x{K}")


def test_every_edge_and_guarded_kernel_on_tiny_tails(handle):
    """Sizes below one tile and one K step, and one past them, on every
    instance that takes ragged sizes (edge instances: only a partial K step,
    or one whole step plus one)."""
    for k in (k for k in KERNELS if k["mode"] != sg.SGEMM_MODE_ALIGNED
              and k["schedule"] != sg.SGEMM_SCHEDULE_SMALL_M):
        handle.set_kernel(k["id"])
        for i, (M, N, K) in enumerate([(1, 1, 1), (k["bm"] - 1, k["bn"] + 1, k["bk"] - 1),
                                       (k["bm"] + 1, k["bn"] - 1, k["bk"] + 1),
                                       (3, 70, 33), (k["bm"] + 5, 2 * k["bn"] - 3, k["bk"])]):
            M, N = edge_fit(k, M, N)
            ta, tb = bool(k["transa"]), bool(k["transb"])
            w = wl.Workload("tail", 4000 + i, M, N, K, 1.0, 1.0, "int4")
            ops = wl.operands(w, lda=(M if ta else K) + 1, ldb=(K if tb else N) + 2,
                              ldc=N + 3, ta=ta, tb=tb)
            gu.check_full(ops, gu.run(handle, ops), exact=True,
                          what=f"{k['name']} {M}x{N}x{K}")


def test_edge_kernels_with_straddling_pieces(handle):
    """Extents along which 16-byte pieces run (N for B as stored, M for A^T)
    two past a multiple of 4, K exactly two K steps and no row padding: the
    first step's direct loads read pieces that straddle the edge, and the
    last step (which holds the last K row) goes through registers."""
    for k in (k for k in KERNELS if k["mode"] == sg.SGEMM_MODE_EDGE
              and k["schedule"] != sg.SGEMM_SCHEDULE_SMALL_M):
        handle.set_kernel(k["id"])
        ta, tb = bool(k["transa"]), bool(k["transb"])
        M, N, K = k["bm"] + 6, k["bn"] + 6, 2 * k["bk"]
        w = wl.Workload("straddle", 4100 + k["id"], M, N, K, 1.0, 1.0, "int4")
        ops = wl.operands(w, ta=ta, tb=tb)  # minimal leading dimensions
        gu.check_full(ops, gu.run(handle, ops), exact=True,
                      what=f"{k['name']} {M}x{N}x{K}")


def test_empty_problems_touch_nothing(handle):
    for M, N in ((0, 16), (16, 0), (0, 0)):
        C = torch.full((64,), 7.0, device="cuda")
        A = torch.ones(256, device="cuda")
        B = torch.ones(256, device="cuda")
        handle.gemm(A, B, C, 1.0, 0.0, M=M, N=N, K=8, lda=8, ldb=max(N, 1),
                    ldc=max(N, 1))
        torch.cuda.synchronize()
        assert torch.all(C == 7.0)


def test_k_zero(handle):
    w = wl.Workload("k0", 5001, 37, 45, 0, 1.0, -2.0, "uniform")
    ops = wl.operands(w)
    out = gu.run(handle, ops)
    got = gu.window(out, 37, 45, 45)
    assert np.array_equal(got, (np.float32(-2.0) * gu.window(ops.C, 37, 45, 45)))
    w = wl.Workload("k0", 5002, 37, 45, 0, 1.0, 0.0, "uniform", "nan")
    ops = wl.operands(w)
    got = gu.window(gu.run(handle, ops), 37, 45, 45)
    assert np.array_equal(got, np.zeros((37, 45), np.float32))


def test_alpha_zero_beta_one_keeps_c(handle):
    w = wl.Workload("ab", 5003, 300, 260, 40, 0.0, 1.0, "uniform")
    ops = wl.operands(w)
    got = gu.window(gu.run(handle, ops), 300, 260, 260)
    assert np.array_equal(got, gu.window(ops.C, 300, 260, 260))


def test_precision_canary(handle):
    """K <= 4, B = 1, A = 1 + m*2^-23: a product path with fewer than 24
    mantissa bits errs by >= 2^-12 per term, far above the bound (<= 2^-18)."""
    rng = np.random.default_rng(77)
    for variant in (sg.SGEMM_VARIANT_MFMA, sg.SGEMM_VARIANT_VALU):
        handle.set_variant(variant)
        for K in (1, 2, 3, 4):
            M, N = 96, 80
            m = rng.integers(1, 2 ** 23, size=(M, K)) | 0x7FF  # low bits set
            a = (1.0 + m * 2.0 ** -23).astype(np.float32)
            b = np.ones((K, N), np.float32)
            c = np.full((M, N), np.nan, np.float32)
            ops = wl.Operands(M, N, K, 1.0, 0.0, a.reshape(-1), K, b.reshape(-1), N,
                              c.reshape(-1), N)
            out = gu.run(handle, ops)
            gu.check_full(ops, out, what=f"canary K={K}")
            if K == 1:
                assert np.array_equal(gu.window(out, M, N, N), np.repeat(a, N, axis=1))


def test_strided_operands_and_sentinels(handle):
    """lda/ldb/ldc beyond the minimum: NaN padding of A and B must not leak
    into the result and the padding of C must stay as it was."""
    w = wl.Workload("strided", 5004, 513, 301, 129, 1.5, 0.5, "uniform")
    ops = wl.operands(w, lda=129 + 7, ldb=301 + 11, ldc=301 + 13)
    gu.check_full(ops, gu.run(handle, ops), what="strided")
    # aligned sizes with padded leading dimensions (multiples of 4) stay aligned
    w = wl.Workload("strided", 5005, 512, 512, 256, 1.0, 0.0, "int4")
    ops = wl.operands(w, lda=256 + 4, ldb=512 + 8, ldc=512 + 12)
    gu.check_full(ops, gu.run(handle, ops), exact=True, what="strided aligned")


@pytest.mark.parametrize("case", ["rows_past_2_31", "tile_span_past_4_gib"])
def test_large_strides(handle, case):
    """Leading dimensions far beyond the sizes: row offsets past 2^31 elements
    in A and C (64-bit addressing), and a stride so large that one K step of
    any MFMA tile spans more than 4 GiB, which the host sends to the guarded
    instance (direct loads use 32-bit lane offsets).  Only the used windows of
    the multi-GiB buffers are written; C's padding must stay untouched."""
    if case == "rows_past_2_31":
        M, N, K = 4100, 256, 96
        lda, ldb, ldc = (1 << 19) + 3, N + 7, (1 << 19) + 1
    else:
        M, N, K = 70, 160, 40
        lda, ldb, ldc = (1 << 25) + (1 << 22) + 3, N, N + 5
    w = wl.Workload("big", 5100 if case == "rows_past_2_31" else 5101, M, N, K, 1.5, 0.5,
                    "int4")
    a = wl.draw(w.cfg_id, wl.ROLE_A, M, K, w.dist)
    b = wl.draw(w.cfg_id, wl.ROLE_B, K, N, w.dist)
    c = wl.draw(w.cfg_id, wl.ROLE_C, M, N, w.dist)
    dev = torch.device("cuda", 0)
    A = torch.empty((M - 1) * lda + K, device=dev)
    B = torch.empty((K - 1) * ldb + N, device=dev)
    C = torch.full(((M - 1) * ldc + N,), float("nan"), device=dev)
    A.as_strided((M, K), (lda, 1)).copy_(torch.from_numpy(a))
    B.as_strided((K, N), (ldb, 1)).copy_(torch.from_numpy(b))
    C.as_strided((M, N), (ldc, 1)).copy_(torch.from_numpy(c))
    sel = sg.sgemm_select_kernel(0, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                                 C.data_ptr(), ldc)
    mode = sg.sgemm_kernel_info(sel)["mode"]
    if case == "rows_past_2_31":
        assert (M - 1) * lda > 2 ** 31 and mode != sg.SGEMM_MODE_GUARDED
    else:
        assert mode == sg.SGEMM_MODE_GUARDED
    handle.gemm(A, B, C, w.alpha, w.beta, M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=ldc)
    torch.cuda.synchronize()
    got = C.as_strided((M, N), (ldc, 1)).cpu().numpy()
    R, T = oracle.gemm(M, N, K, w.alpha, a, K, b, N, w.beta, c, N)
    gu.check(got, R, T, K, w.alpha, w.beta, c, exact=True, what=case)
    if ldc > N:  # padding after a few rows, including the last full one
        width = min(ldc - N, 64)
        for row in (0, M // 2, M - 2):
            pad = C[row * ldc + N: row * ldc + N + width].cpu().numpy()
            assert np.all(np.isnan(pad)), f"{case}: C padding written in row {row}"
    del A, B, C
    torch.cuda.empty_cache()


@pytest.mark.parametrize("tb", [True, False], ids=["b_nk", "b_kn"])
def test_one_pass_large_strides(tb):
    """The one-pass small-M kernels address rows of B and C in 64 bits: row
    offsets past 2^31 elements (B's rows along K or along N, C's rows) give
    the oracle's result, exact on integers, and C's padding stays untouched.
    Only the used windows of the multi-GiB buffers are written."""
    M, N, K = 3, 40, 300
    name = "valu_S4_nt_small" if tb else "valu_S4x32_small"
    ldb = (1 << 26) + 5 if tb else (1 << 23) + 3
    lda, ldc = K + 1, (1 << 30) + 3
    w = wl.Workload("bigsmall", 5200 + int(tb), M, N, K, 1.5, 0.5, "int4")
    a = wl.draw(w.cfg_id, wl.ROLE_A, M, K, w.dist)
    b = wl.draw(w.cfg_id, wl.ROLE_B, K, N, w.dist)  # B(k, n)
    c = wl.draw(w.cfg_id, wl.ROLE_C, M, N, w.dist)
    dev = torch.device("cuda", 0)
    rows_b, cols_b = (N, K) if tb else (K, N)
    assert (rows_b - 1) * ldb > 2 ** 31 and (M - 1) * ldc > 2 ** 31
    A = torch.empty((M - 1) * lda + K, device=dev)
    B = torch.empty((rows_b - 1) * ldb + cols_b, device=dev)
    C = torch.full(((M - 1) * ldc + N,), float("nan"), device=dev)
    A.as_strided((M, K), (lda, 1)).copy_(torch.from_numpy(a))
    B.as_strided((rows_b, cols_b), (ldb, 1)).copy_(torch.from_numpy(b.T.copy() if tb else b))
    C.as_strided((M, N), (ldc, 1)).copy_(torch.from_numpy(c))
    h = sg.Handle(workspace=False)
    try:
        h.set_kernel({k["name"]: k["id"] for k in KERNELS}[name])
        h.gemm(A, B, C, w.alpha, w.beta, M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=ldc,
               transb=tb)
        torch.cuda.synchronize()
    finally:
        h.close()
    got = C.as_strided((M, N), (ldc, 1)).cpu().numpy()
    R, T = oracle.gemm(M, N, K, w.alpha, a, K, b, N, w.beta, c, N)
    gu.check(got, R, T, K, w.alpha, w.beta, c, exact=True, what=name)
    pad = C[N: N + 64].cpu().numpy()
    assert np.all(np.isnan(pad)), f"{name}: C padding written"
    del A, B, C
    torch.cuda.empty_cache()


def test_misaligned_base_pointers(handle):
    w = wl.Workload("mis", 5006, 256, 256, 256, 1.0, 0.0, "int4")
    ops = wl.operands(w)
    A, B, C = gu.to_device(ops)
    A1 = torch.empty(A.numel() + 1, device="cuda")
    A1[1:] = A
    B1 = torch.empty(B.numel() + 3, device="cuda")
    B1[3:] = B
    sel = sg.sgemm_select_kernel(0, 256, 256, 256, A1[1:].data_ptr(), 256,
                                 B1[3:].data_ptr(), 256, C.data_ptr(), 256)
    # MFMA direct loads need only 4-byte aligned operands
    assert sg.sgemm_kernel_info(sel)["mode"] == sg.SGEMM_MODE_ALIGNED
    out = gu.run(handle, ops, dev=(A1[1:], B1[3:], C))
    gu.check_full(ops, out, exact=True, what="misaligned")


@pytest.mark.parametrize("shape", [(48, 4096, 4096), (64, 4096, 4096), (100, 1000, 3000),
                                   (256, 256, 16384), (512, 512, 8192)])
def test_stream_k_plans(handle, shape):
    """Few output tiles over a long K (M past the small-M kernels' 32 rows,
    or a small C with a deep contraction) leave most CUs idle with one
    tile per workgroup, so the
    planner runs them stream-K when the handle has a workspace: integer
    inputs, so the split-and-added tiles must still be bit-exact, and two
    runs must agree bit for bit."""
    M, N, K = shape
    w = wl.Workload("sk", 6000 + M % 97 + N % 89, M, N, K, 1.5, 0.5, "int4")
    ops = wl.operands(w)
    A, B, C = gu.to_device(ops)
    plan = handle.plan(M, N, K, A.data_ptr(), ops.lda, B.data_ptr(), ops.ldb,
                       C.data_ptr(), ops.ldc)
    assert any(sg.sgemm_kernel_schedule(k) == sg.SGEMM_SCHEDULE_STREAM_K
               for k, _, _ in plan), [sg.sgemm_kernel_name(k) for k, _, _ in plan]
    out = gu.run(handle, ops, dev=(A, B, C))
    gu.check_full(ops, out, exact=True, what=f"stream-K {shape}")
    C.copy_(torch.from_numpy(ops.C).cuda())
    again = gu.run(handle, ops, dev=(A, B, C))
    assert np.array_equal(out.view(np.uint32), again.view(np.uint32))


def test_stream_k_uniform_values(handle):
    """Uniform values through a stream-K plan on a ragged shape: within the
    FP32 bound."""
    w = wl.Workload("sku", 6101, 90, 2001, 3001, 1.0, 1.0, "uniform")
    ops = wl.operands(w)
    A, B, C = gu.to_device(ops)
    plan = handle.plan(w.M, w.N, w.K, A.data_ptr(), ops.lda, B.data_ptr(), ops.ldb,
                       C.data_ptr(), ops.ldc)
    assert [sg.sgemm_kernel_schedule(k) for k, _, _ in plan] == [sg.SGEMM_SCHEDULE_STREAM_K]
    gu.check_full(ops, gu.run(handle, ops, dev=(A, B, C)), what="stream-K uniform")


@pytest.mark.parametrize("name", ["c1_128", "c2_1024", "c3_4096", "c4_edge", "c5_mlp"])
def test_benchmark_problems_never_use_the_workspace(handle, name):
    """The five benchmark problems plan one-tile-per-workgroup launches even
    on a handle with a workspace, in every operand storage: the workspace is
    never touched for them."""
    w = W[name]
    assert handle.workspace is not None
    for ta in (False, True):
        for tb in (False, True):
            lda = w.M if ta else w.K
            ldb = w.K if tb else w.N
            plan = handle.plan(w.M, w.N, w.K, 0x10000000, lda, 0x20000000, ldb,
                               0x40000000, w.N, transa=ta, transb=tb)
            assert all(sg.sgemm_kernel_schedule(k) == sg.SGEMM_SCHEDULE_TILES
                       for k, _, _ in plan), (name, ta, tb, plan)


def test_clocked_run_matches_and_reads_a_clock(handle):
    """sgemm_diag_run_clocked runs the same plan as sgemm_run (bit-identical
    output), stamps every workgroup, and reads a shader clock in a plausible
    range; plans that are not one tile-per-workgroup MFMA launch are refused
    before anything runs."""
    w = wl.Workload("clk", 5300, 1024, 768, 512, 1.5, 0.5, "uniform")
    ops = wl.operands(w)
    A, B, C = gu.to_device(ops)
    c0 = C.clone()
    ref = gu.run(handle, ops, dev=(A, B, C))
    C.copy_(c0)
    ghz, span_us = handle.gemm_clocked(A, B, C, w.alpha, w.beta, M=w.M, N=w.N, K=w.K,
                                       lda=ops.lda, ldb=ops.ldb, ldc=ops.ldc)
    torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    assert 0.5 < ghz < 3.5 and 0 < span_us < 1e5, (ghz, span_us)
    assert 1000 < sg.sgemm_diag_wall_clock_khz() < 10 ** 7
    stamps = torch.zeros(4 * 8, dtype=torch.int64, device="cuda")
    with pytest.raises(sg.SgemmError) as e:  # more workgroups than slots
        sg.sgemm_diag_run_clocked(handle.h, 0, 0, w.M, w.N, w.K, 1.0, A.data_ptr(), ops.lda,
                                  B.data_ptr(), ops.ldb, 0.0, C.data_ptr(), ops.ldc,
                                  stamps.data_ptr(), 8)
    assert e.value.status == sg.SGEMM_ERR_SIZE
    # one row of C plans a stream-K or small-M launch, not tiles
    plan = handle.plan(1, w.N, w.K, A.data_ptr(), ops.lda, B.data_ptr(), ops.ldb,
                       C.data_ptr(), ops.ldc)
    assert sg.sgemm_kernel_schedule(plan[0][0]) != sg.SGEMM_SCHEDULE_TILES
    with pytest.raises(sg.SgemmError) as e:
        sg.sgemm_diag_run_clocked(handle.h, 0, 0, 1, w.N, w.K, 1.0, A.data_ptr(), ops.lda,
                                  B.data_ptr(), ops.ldb, 0.0, C.data_ptr(), ops.ldc,
                                  stamps.data_ptr(), 8)
    assert e.value.status == sg.SGEMM_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(stamps == 0)


def test_no_workspace_no_stream_k():
    """Without a workspace no stream-K kernel is planned, and a forced one is
    refused before anything is launched."""
    h = sg.Handle(workspace=False)
    try:
        M, N, K = 1000, 1500, 777
        A = torch.ones(M * K, device="cuda")
        B = torch.ones(K * N, device="cuda")
        C = torch.full((M * N,), 3.0, device="cuda")
        plan = h.plan(M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(), N)
        assert all(sg.sgemm_kernel_schedule(k) == sg.SGEMM_SCHEDULE_TILES for k, _, _ in plan)
        sk = next(k for k in KERNELS if k["schedule"] == sg.SGEMM_SCHEDULE_STREAM_K
                  and k["mode"] == sg.SGEMM_MODE_EDGE and not k["transa"] and not k["transb"])
        h.set_kernel(sk["id"])
        with pytest.raises(sg.SgemmError) as e:
            h.gemm(A, B, C, 1.0, 1.0, M=M, N=N, K=K, lda=K, ldb=N, ldc=N)
        assert e.value.status == sg.SGEMM_ERR_UNSUPPORTED
        torch.cuda.synchronize()
        assert torch.all(C == 3.0)
    finally:
        h.close()


SMALL_M = [k for k in KERNELS if k["schedule"] == sg.SGEMM_SCHEDULE_SMALL_M
           and k["variant"] == sg.SGEMM_VARIANT_VALU]
MFMA_SPLIT_K = [k for k in KERNELS if k["schedule"] == sg.SGEMM_SCHEDULE_SMALL_M
                and k["variant"] == sg.SGEMM_VARIANT_MFMA]


@pytest.mark.parametrize("k", MFMA_SPLIT_K, ids=[k["name"] for k in MFMA_SPLIT_K])
def test_mfma_split_k_kernels(k):
    """The small-M kernels on the matrix cores (one tile row, K split over
    workgroups, partial sums in the workspace), forced: 1 row (4 when A is
    stored K x M), a ragged row count and bm rows; N short of, at and past a
    tile and not a multiple of 4; K below one K step, ragged, and long enough
    for many ranges; padded leading dimensions; integers exact, uniform
    values within the bound.  Without a workspace they are refused."""
    h = sg.Handle()
    try:
        h.set_kernel(k["id"])
        ta, tb = bool(k["transa"]), bool(k["transb"])
        m_small = 4 if ta else 1
        cases = [(m_small, 37, 7), (k["bm"] // 2 + 1, 300, 1025), (k["bm"], 64, 4111),
                 (m_small, 4098, 3000), (k["bm"], 1000, 777)]
        for i, (M, N, K) in enumerate(cases):
            for dist in ("int4", "uniform"):
                w = wl.Workload("mfsk", 7600 + 10 * i + k["id"], M, N, K, 1.5, -0.5, dist)
                ops = wl.operands(w, lda=(M if ta else K) + 3, ldb=(K if tb else N) + 1,
                                  ldc=N + 2, ta=ta, tb=tb)
                gu.check_full(ops, gu.run(h, ops), exact=(dist == "int4"),
                              what=f"{k['name']} {M}x{N}x{K} {dist}")
        h.set_workspace(0)
        ops = wl.operands(wl.Workload("mfsk", 7700, k["bm"], 300, 1025, 1.0, 1.0, "int4"),
                          ta=ta, tb=tb)
        A, B, C = gu.to_device(ops)
        c0 = C.clone()
        with pytest.raises(sg.SgemmError) as e:
            h.gemm(A, B, C, 1.0, 1.0, M=ops.M, N=ops.N, K=ops.K, lda=ops.lda, ldb=ops.ldb,
                   ldc=ops.ldc, transa=ta, transb=tb)
        assert e.value.status == sg.SGEMM_ERR_UNSUPPORTED
        torch.cuda.synchronize()
        assert torch.equal(C, c0)
    finally:
        h.close()


@pytest.mark.parametrize("k", SMALL_M, ids=[k["name"] for k in SMALL_M])
@pytest.mark.parametrize("workspace", [True, False], ids=["ws", "nows"])
def test_split_k_kernels(k, workspace):
    """Every small-M kernel on ragged sizes: 1 and bm rows, columns short of,
    at and past a workgroup's block and not a multiple of 4, K below, at and
    past one staged chunk of A (B as stored) or one 256-k piece and a run of
    several per wave (B transposed) and not a multiple of 4, padded leading
    dimensions; integer inputs (exact) and uniform ones (bound).  B as
    stored: with a workspace K is split over workgroups and a second kernel
    adds the ranges, without one a single range runs (B transposed needs no
    workspace either way)."""
    h = sg.Handle(workspace=workspace)
    try:
        h.set_kernel(k["id"])
        ta, tb = bool(k["transa"]), bool(k["transb"])
        cases = [(1, 1, 1), (k["bm"], 3, 7), (k["bm"] - 1, 255, 300), (1, 257, 1025),
                 (k["bm"], 1000, 777), (k["bm"], 4096, 2048), (2, 33, 2049)]
        for i, (M, N, K) in enumerate(cases):
            M = min(max(M, 1), k["bm"])
            for dist in ("int4", "uniform"):
                w = wl.Workload("skinny", 7000 + 10 * i + k["id"], M, N, K, 1.5, -0.5, dist)
                ops = wl.operands(w, lda=(M if ta else K) + 3, ldb=(K if tb else N) + 1,
                                  ldc=N + 2, ta=ta, tb=tb)
                gu.check_full(ops, gu.run(h, ops), exact=(dist == "int4"),
                              what=f"{k['name']} ws={workspace} {M}x{N}x{K} {dist}")
    finally:
        h.close()


@pytest.mark.parametrize("tb,shape", [(False, (1, 4096, 4096)), (False, (16, 4096, 4096)),
                                      (False, (7, 11008, 4096)), (False, (16, 2000, 8192)),
                                      (True, (1, 4096, 4096)), (True, (4, 4096, 4096)),
                                      (True, (3, 11008, 4096)), (True, (2, 4096, 16384)),
                                      (True, (6, 4096, 4096)), (True, (8, 14336, 4096))])
def test_split_k_plans(handle, shape, tb):
    """Decode-like shapes (a few rows of A against a large B, stored K x N or
    N x K) plan the small-M kernel; bit-exact on integer inputs, bitwise
    repeatable, and within the bound on normal(0, 0.02) inputs."""
    M, N, K = shape
    w = wl.Workload("skinnyplan", 7100 + M + N % 97, M, N, K, 1.0, 1.0, "int4")
    ops = wl.operands(w, tb=tb)
    A, B, C = gu.to_device(ops)
    plan = handle.plan(M, N, K, A.data_ptr(), ops.lda, B.data_ptr(), ops.ldb,
                       C.data_ptr(), ops.ldc, transb=int(tb))
    assert [sg.sgemm_kernel_schedule(k) for k, _, _ in plan] == [sg.SGEMM_SCHEDULE_SMALL_M]
    out = gu.run(handle, ops, dev=(A, B, C))
    gu.check_full(ops, out, exact=True, what=f"small-M plan {shape} tb={tb}")
    C.copy_(torch.from_numpy(ops.C).cuda())
    again = gu.run(handle, ops, dev=(A, B, C))
    assert np.array_equal(out.view(np.uint32), again.view(np.uint32))
    w = wl.Workload("skinnyplan", 7200 + M, M, N, K, 1.0, 0.0, "normal", "nan")
    ops = wl.operands(w, tb=tb)
    gu.check_full(ops, gu.run(handle, ops), what=f"split-K plan {shape} normal")


@pytest.mark.parametrize("shape,tb,want", [((1, 4096, 4096), True, "valu_S1_nt_small"),
                                           ((2, 4096, 4096), True, "valu_S2_nt_small"),
                                           ((4, 11008, 4096), True, "valu_S4_nt_small"),
                                           ((8, 4096, 4096), True, "valu_S8_nt_small"),
                                           ((16, 4096, 4096), True, "mfma_M32x64_nt_splitk_edge"),
                                           ((1, 4096, 4096), False, "valu_S1x32_small"),
                                           ((16, 4096, 4096), False, "mfma_M32x64_splitk_edge")])
def test_one_pass_plans(handle, shape, tb, want):
    """With a workspace, the planner takes the one-pass vector-ALU kernels
    where they measured faster than split K on the matrix cores (B stored N
    x K up to 8 rows: 1 x 4096 x 4096 11.9 against 16.0 us; B stored K x N:
    13.2-13.7 against 16.9), and split K past their rows; the planned call is
    exact on integers."""
    M, N, K = shape
    w = wl.Workload("onepass", 7300 + M, M, N, K, 1.0, 0.5, "int4")
    ops = wl.operands(w, tb=tb)
    A, B, C = gu.to_device(ops)
    plan = handle.plan(M, N, K, A.data_ptr(), ops.lda, B.data_ptr(), ops.ldb,
                       C.data_ptr(), ops.ldc, transb=tb)
    assert [sg.sgemm_kernel_name(k) for k, _, _ in plan] == [want]
    gu.check_full(ops, gu.run(handle, ops, dev=(A, B, C)), exact=True,
                  what=f"one-pass plan {shape} tb={tb}")


@pytest.mark.parametrize("ta", [False, True])
def test_one_pass_without_workspace(ta):
    """A handle with no workspace (as sgemm_create gives) plans the one-pass
    kernel for a few rows against B stored K x N, where split K cannot run;
    uniform inputs within the bound, integers exact."""
    h = sg.Handle(workspace=False)
    try:
        for M, N, K in ((1, 4096, 4096), (3, 1000, 777), (4, 2050, 4100)):
            w = wl.Workload("onepassnows", 7400 + M, M, N, K, 1.5, -0.5, "uniform")
            ops = wl.operands(w, ta=ta)
            A, B, C = gu.to_device(ops)
            plan = h.plan(M, N, K, A.data_ptr(), ops.lda, B.data_ptr(), ops.ldb,
                          C.data_ptr(), ops.ldc, transa=ta)
            names = [sg.sgemm_kernel_name(k) for k, _, _ in plan]
            assert len(names) == 1 and "x32_" in names[0] and "small" in names[0], names
            gu.check_full(ops, gu.run(h, ops, dev=(A, B, C)), what=f"{names} {M}x{N}x{K}")
            w = wl.Workload("onepassnows", 7500 + M, M, N, K, 1.0, 1.0, "int4")
            ops = wl.operands(w, ta=ta)
            gu.check_full(ops, gu.run(h, ops), exact=True, what=f"{names} {M}x{N}x{K} int")
    finally:
        h.close()


def random_problems(seed, count):
    """Seeded random problems that reach every kind of plan: small M against
    wide B, ragged and aligned sizes around the tile edges, deep K with few
    tiles, large M and N (the big tiles, split plans) with a short K, every
    operand storage, padded leading dimensions, varied alpha and beta (beta
    = 0 with a NaN-filled C)."""
    rng = np.random.default_rng(seed)
    picks = []
    for i in range(count):
        kind = i % 5
        if kind == 0:    # small M
            M = int(rng.integers(1, 17))
            N = int(rng.integers(1, 5000))
            K = int(rng.integers(1, 4000))
        elif kind == 1:  # around tile multiples
            M = int(rng.choice([64, 128, 256])) * int(rng.integers(1, 6)) + int(rng.integers(-3, 4))
            N = int(rng.choice([64, 128, 256])) * int(rng.integers(1, 6)) + int(rng.integers(-3, 4))
            K = int(rng.choice([16, 32, 64])) * int(rng.integers(1, 24)) + int(rng.integers(-2, 3))
        elif kind == 2:  # few tiles, deep K
            M = int(rng.integers(17, 300))
            N = int(rng.integers(17, 300))
            K = int(rng.integers(1000, 6000))
        elif kind == 3:  # large M and N, short K
            M = int(rng.integers(1500, 4200))
            N = int(rng.integers(1500, 4200))
            K = int(rng.integers(16, 160))
        else:            # anything up to mid sizes
            M, N, K = (int(x) for x in rng.integers(1, 1200, size=3))
        M, N, K = max(M, 1), max(N, 1), max(K, 1)
        ta, tb = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
        alpha = float(rng.choice([1.0, -1.5, 0.5]))
        beta = float(rng.choice([0.0, 1.0, -0.5]))
        pads = [int(x) for x in rng.integers(0, 5, size=3)]
        picks.append((M, N, K, ta, tb, alpha, beta, pads))
    return picks


@pytest.mark.parametrize("chunk", range(4))
def test_random_problems_integer_exact(handle, chunk):
    """60 seeded random problems through the planner (with a workspace, so
    stream-K and the small-M kernels are candidates): bit-exact on integer
    inputs, the padding of C untouched."""
    for i, (M, N, K, ta, tb, alpha, beta, pads) in enumerate(random_problems(8100 + chunk, 15)):
        w = wl.Workload("rand", 8200 + 16 * chunk + i, M, N, K, alpha, beta, "int4",
                        "nan" if beta == 0.0 else "dist")
        ops = wl.operands(w, lda=(M if ta else K) + pads[0], ldb=(K if tb else N) + pads[1],
                          ldc=N + pads[2], ta=ta, tb=tb)
        plan = handle.plan(M, N, K, 0x10000000, ops.lda, 0x20000000, ops.ldb, 0x40000000,
                           ops.ldc, transa=ta, transb=tb)
        what = (f"{M}x{N}x{K} ta={ta} tb={tb} a={alpha} b={beta} pads={pads} "
                f"plan={[sg.sgemm_kernel_name(k) for k, _, _ in plan]}")
        print(what, flush=True)
        gu.check_full(ops, gu.run(handle, ops), exact=True, what=what)


def test_deterministic(handle):
    ops = wl.operands(wl.Workload("det", 2, 1024, 1024, 1024, 1.0, 0.0, "uniform"))
    A, B, C = gu.to_device(ops)
    outs = []
    for _ in range(3):
        C.fill_(0.0)
        handle.gemm(A, B, C, 1.0, 0.0, M=1024, N=1024, K=1024, lda=1024, ldb=1024,
                    ldc=1024)
        torch.cuda.synchronize()
        outs.append(C.cpu().numpy().view(np.uint32).copy())
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_runs_on_a_side_stream(handle):
    w = wl.Workload("stream", 5007, 384, 512, 96, 1.0, 1.0, "int4")
    ops = wl.operands(w)
    dev = gu.to_device(ops)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    out = gu.run(handle, ops, dev=dev, stream=s)
    gu.check_full(ops, out, exact=True, what="side stream")


def test_errors_launch_nothing(handle):
    A = torch.ones(64 * 64, device="cuda")
    B = torch.ones(64 * 64, device="cuda")
    with pytest.raises(sg.SgemmError) as e:
        handle.gemm(A, B, A, 1.0, 0.0, M=64, N=64, K=64, lda=64, ldb=64, ldc=64)
    assert e.value.status == sg.SGEMM_ERR_ALIAS
    with pytest.raises(sg.SgemmError) as e:
        handle.gemm(A, B, torch.ones(64 * 64, device="cuda"), 1.0, 0.0, M=64, N=64,
                    K=64, lda=63, ldb=64, ldc=64)
    assert e.value.status == sg.SGEMM_ERR_LD
    aligned = [k for k in KERNELS if k["mode"] == sg.SGEMM_MODE_ALIGNED][0]
    handle.set_kernel(aligned["id"])
    C = torch.ones(64 * 64, device="cuda")
    with pytest.raises(sg.SgemmError) as e:
        handle.gemm(A, B, C, 1.0, 0.0, M=63, N=64, K=64, lda=64, ldb=64, ldc=64)
    assert e.value.status == sg.SGEMM_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(C == 1.0)
