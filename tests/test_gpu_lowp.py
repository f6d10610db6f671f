"""Parity of the HIP product with 16-bit A and B (bfloat16 / binary16) or
8-bit A and B (OCP E4M3 / E5M2) and FP32 C, through the C ABI, with the FP64
CPU oracle on the same bit patterns (the gsyq.cn guide, section 5.1:
low-precision inputs, FP32 accumulation).

Acceptance is that of the FP32 product: every product of two 16-bit (or
8-bit) values is exact in FP32, so |C_gpu - r| <= 4*max(K,1)*2^-24*(|alpha|*t + |beta*c|)
elementwise against the unrounded FP64 r of the stored 16-bit values, and
bit-exact results for integer inputs (every partial sum an integer below
2^24, which an accumulator narrower than FP32 would not keep at these K).
The 8-bit kernels' matrix instruction sums each block of 64 products in a
narrower fixed-point window whose rounding is not documented: for them the
random-input checks are an envelope (the FP32 bound plus a per-block
allowance, ``gpu_util.FP8_BLOCK_ALLOWANCE``, measured here by
``test_fp8_envelope_measurement``), and the parity evidence is the integer
tests, which stay bit-exact.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import fp32_gemm_major_amd as sg  # noqa: E402
from fp32_gemm_major_amd import workloads as wl  # noqa: E402
from tests import gpu_util as gu  # noqa: E402

W = wl.WORKLOADS
FORMATS = wl.FORMATS16


@pytest.fixture(scope="module")
def handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h = sg.Handle(workspace=False)
    yield h
    h.close()


@pytest.fixture(autouse=True)
def _auto_kernel(handle):
    handle.set_lowp_kernel(-1)
    yield
    handle.set_lowp_kernel(-1)


ALL_KERNELS = [] if not __import__("os").path.exists(sg.LIBRARY) else sg.lowp_kernel_table()
# one-tile-per-workgroup kernels (the split-K ones need a workspace: below)
KERNELS = [k for k in ALL_KERNELS if k["schedule"] == sg.SGEMM_SCHEDULE_TILES]
SPLIT_K = [k for k in ALL_KERNELS if k["schedule"] == sg.SGEMM_SCHEDULE_SMALL_M
           and "_sk_" in k["name"]]
# one-pass matrix-core kernels for at most 16 rows of A, B stored N x K
GEMV = [k for k in ALL_KERNELS if "_G16x16_" in k["name"]]
DT_NAME = {sg.SGEMM_DTYPE_BF16: "bf16", sg.SGEMM_DTYPE_F16: "f16",
           sg.SGEMM_DTYPE_FP8_E4M3: "fp8e4m3", sg.SGEMM_DTYPE_FP8_E5M2: "fp8e5m2"}
FORMATS8 = wl.FORMATS8


@pytest.mark.parametrize("k", KERNELS, ids=[k["name"] for k in KERNELS])
@pytest.mark.parametrize("dist", ["uniform", "int4"])
def test_each_kernel(handle, k, dist):
    """Every kernel of the table on a problem of several tiles (guarded
    kernels: ragged sizes, odd leading dimensions, a partial K step)."""
    handle.set_lowp_kernel(k["id"])
    ta, tb = bool(k["transa"]), bool(k["transb"])
    if k["mode"] == sg.SGEMM_MODE_ALIGNED:
        M, N, K = 2 * k["bm"], 3 * k["bn"], 4 * k["bk"]
        pad_a, pad_b, ldc = 8, 16, N + 4
    else:
        M, N, K = 2 * k["bm"] + 37, k["bn"] + 19, 3 * k["bk"] + 5
        pad_a, pad_b, ldc = 3, 1, N + 5
    lda = (M if ta else K) + pad_a
    ldb = (K if tb else N) + pad_b
    w = wl.Workload("case", 700 + k["id"], M, N, K, 1.5, 0.5, dist)
    ops = wl.operands16(w, DT_NAME[k["dtype"]], lda=lda, ldb=ldb, ldc=ldc, ta=ta, tb=tb)
    out = gu.run16(handle, ops)
    gu.check_full16(ops, out, exact=(dist == "int4"), what=k["name"])


# ---- the benchmark's workloads with 16-bit A and B ---------------------------

@pytest.mark.parametrize("dt", FORMATS)
@pytest.mark.parametrize("name", ["c1_128", "c1_128_int", "c2_1024", "c4_edge",
                                  "c4_edge_int"])
def test_small_workloads_full(handle, dt, name):
    ops = wl.operands16(W[name], dt)
    out = gu.run16(handle, ops)
    gu.check_full16(ops, out, exact=W[name].dist == "int4", what=f"{name} {dt}")


@pytest.mark.parametrize("dt", FORMATS)
@pytest.mark.parametrize("name", ["c3_4096", "c3_4096_int", "c5_mlp"])
def test_large_workloads_sampled(handle, dt, name):
    ops = wl.operands16(W[name], dt)
    out = gu.run16(handle, ops)
    rows = gu.edge_rows(ops.M, extra=4)[:10]
    cols = [0, 1, 127, 128, 255, 256, ops.N // 2, ops.N - 1]
    gu.check_sampled16(ops, out, rows, cols, exact=W[name].dist == "int4",
                       what=f"{name} {dt}")


@pytest.mark.parametrize("ta,tb", [(True, False), (False, True), (True, True)],
                         ids=["tn", "nt", "tt"])
@pytest.mark.parametrize("dt", FORMATS)
def test_transposed_4096_sampled(handle, dt, ta, tb):
    ops = wl.operands16(W["c3_4096"], dt, ta=ta, tb=tb)
    out = gu.run16(handle, ops)
    gu.check_sampled16(ops, out, [0, 255, 256, 2047, 4095], [0, 256, 4095],
                       npoints=2048, what=f"4096 {dt} ta={ta} tb={tb}")


# ---- edge cases ----------------------------------------------------------------

@pytest.mark.parametrize("dt", FORMATS)
def test_tiny_sizes_integer_exact(handle, dt):
    rng = np.random.default_rng(61)
    for case in range(40):
        M, N, K = (int(x) for x in rng.integers(1, 71, size=3))
        ta, tb = bool(case & 1), bool(case & 2)
        w = wl.Workload("tiny", 3000 + case, M, N, K, 1.0, 1.0, "int4")
        ops = wl.operands16(w, dt, ta=ta, tb=tb)
        out = gu.run16(handle, ops)
        gu.check_full16(ops, out, exact=True, what=f"tiny {dt} {M}x{N}x{K} {ta}{tb}")


@pytest.mark.parametrize("dt", FORMATS + FORMATS8)
def test_nan_c_with_beta_zero(handle, dt):
    ops = wl.operands16(W["c2_1024"], dt, M=300, N=260, K=200, tb=dt in FORMATS8)
    assert np.isnan(ops.C).all()
    out = gu.run16(handle, ops)
    gu.check_full16(ops, out, what="beta 0 with NaN C")


@pytest.mark.parametrize("dt", FORMATS + FORMATS8)
def test_k_zero_and_empty(handle, dt):
    w = W["c4_edge"]
    tb = dt in FORMATS8
    ops = wl.operands16(w, dt, M=70, N=50, K=0, ldc=53, tb=tb)
    out = gu.run16(handle, ops)
    gu.check_full16(ops, out, what="K = 0")  # C = beta * C
    for M, N in ((0, 50), (70, 0)):
        ops = wl.operands16(w, dt, M=M, N=N, K=16, tb=tb)
        A, B, C = gu.to_device16(ops)
        before = C.clone()
        handle.gemm_lowp(A, B, C, 1.0, 1.0, M=M, N=N, K=16, lda=ops.lda, ldb=ops.ldb,
                         ldc=ops.ldc, transb=tb)
        torch.cuda.synchronize()
        assert torch.equal(before.view(torch.int32), C.view(torch.int32))


@pytest.mark.parametrize("dt", FORMATS)
def test_misaligned_operands_and_sentinels(handle, dt):
    """A and B starting one element past a 16-byte boundary, odd leading
    dimensions and padded C: the guarded kernels, element loads, untouched
    C padding (NaN-filled padding in A and B never reaches an output)."""
    w = wl.Workload("mis", 77, 300, 270, 150, 1.25, -0.5, "uniform")
    ops = wl.operands16(w, dt, lda=151, ldb=273, ldc=275)
    A, B, C = gu.to_device16(ops)
    t16 = A.dtype
    A1 = torch.empty(A.numel() + 1, dtype=t16, device=A.device)
    A1[1:] = A
    B1 = torch.empty(B.numel() + 1, dtype=t16, device=B.device)
    B1[1:] = B
    out = gu.run16(handle, ops, dev=(A1[1:], B1[1:], C))
    gu.check_full16(ops, out, what="misaligned")


@pytest.mark.parametrize("dt", FORMATS)
def test_alpha_zero_beta_one_keeps_c(handle, dt):
    w = wl.Workload("keep", 78, 256, 256, 128, 0.0, 1.0, "uniform")
    ops = wl.operands16(w, dt)
    out = gu.run16(handle, ops)
    assert np.array_equal(out, ops.C)


def test_deterministic(handle):
    ops = wl.operands16(W["c4_edge"], "bf16")
    dev = gu.to_device16(ops)
    c0 = dev[2].clone()
    first = gu.run16(handle, ops, dev=dev)
    for _ in range(3):
        dev[2].copy_(c0)
        again = gu.run16(handle, ops, dev=dev)
        assert np.array_equal(first.view(np.uint32), again.view(np.uint32))


def test_forced_kernel_that_cannot_run(handle):
    aligned = [k for k in KERNELS if k["mode"] == sg.SGEMM_MODE_ALIGNED and
               k["dtype"] == sg.SGEMM_DTYPE_BF16 and not k["transa"] and
               not k["transb"]][0]
    handle.set_lowp_kernel(aligned["id"])
    ops = wl.operands16(W["c4_edge"], "bf16")
    A, B, C = gu.to_device16(ops)
    with pytest.raises(sg.SgemmError) as e:
        handle.gemm_lowp(A, B, C, 1.0, 1.0, M=ops.M, N=ops.N, K=ops.K, lda=ops.lda,
                         ldb=ops.ldb, ldc=ops.ldc)
    assert e.value.status == sg.SGEMM_ERR_UNSUPPORTED
    # the wrong format is unsupported too
    f16 = [k for k in KERNELS if k["dtype"] == sg.SGEMM_DTYPE_F16][0]
    handle.set_lowp_kernel(f16["id"])
    with pytest.raises(sg.SgemmError):
        handle.gemm_lowp(A, B, C, 1.0, 1.0, M=ops.M, N=ops.N, K=ops.K, lda=ops.lda,
                         ldb=ops.ldb, ldc=ops.ldc)


def test_torch_tensor_shapes(handle):
    """2-D tensors give sizes and leading dimensions; the result matches the
    oracle on the same values."""
    ops = wl.operands16(W["c4_edge"], "f16", M=200, N=136, K=96)
    A, B, C = gu.to_device16(ops)
    A2, B2, C2 = A.view(200, 96), B.view(96, 136), C.view(200, 136)
    handle.gemm_lowp(A2, B2, C2, ops.alpha, ops.beta)
    torch.cuda.synchronize()
    gu.check_full16(ops, C.cpu().numpy(), what="2-D tensors")


@pytest.mark.parametrize("nk", [1, 2, 3, 5])
def test_aligned_kernels_short_k(handle, nk):
    """Aligned kernels with one to five K steps: the software pipeline's
    start and end (steps past the last one repeat it into an unused stage)."""
    for k in KERNELS:
        if k["mode"] != sg.SGEMM_MODE_ALIGNED:
            continue
        handle.set_lowp_kernel(k["id"])
        ta, tb = bool(k["transa"]), bool(k["transb"])
        M, N, K = k["bm"], 2 * k["bn"], nk * k["bk"]
        w = wl.Workload("shortk", 800 + 10 * nk + k["id"] % 10, M, N, K, 1.0, 1.0, "int4")
        ops = wl.operands16(w, DT_NAME[k["dtype"]], ta=ta, tb=tb)
        out = gu.run16(handle, ops)
        gu.check_full16(ops, out, exact=True, what=f"{k['name']} nk={nk}")


@pytest.mark.parametrize("case", ["k_whole_straddle", "k_whole_no_straddle",
                                  "k_piece8_not16", "k_short", "k_one_past"])
def test_edge_kernels_k_cases(handle, case):
    """Edge kernels: K a multiple of the K step with an M or N edge that is not
    a multiple of one 16-byte piece (8 elements of a 16-bit format, 16 of an
    8-bit one: the last whole K step goes through registers), the same with
    multiples of a piece (every step a direct load), K under one step (no
    direct steps at all) and K one past a multiple of 64."""
    M, N, K = {"k_whole_straddle": (150, 133, 256), "k_whole_no_straddle": (160, 144, 256),
               "k_piece8_not16": (152, 136, 256), "k_short": (150, 133, 40),
               "k_one_past": (150, 133, 129)}[case]
    for k in KERNELS:
        if k["mode"] != sg.SGEMM_MODE_EDGE:
            continue
        handle.set_lowp_kernel(k["id"])
        ta, tb = bool(k["transa"]), bool(k["transb"])
        w = wl.Workload("edgek", 850 + k["id"] % 50, M, N, K, 1.5, -0.5, "int4")
        ops = wl.operands16(w, DT_NAME[k["dtype"]], ta=ta, tb=tb,
                            lda=(M if ta else K) + 1, ldb=(K if tb else N) + 3, ldc=N + 2)
        out = gu.run16(handle, ops)
        gu.check_full16(ops, out, exact=True, what=f"{k['name']} {case}")



# ---- 8-bit formats ---------------------------------------------------------------

STORAGES = [(False, True), (False, False), (True, False), (True, True)]
STORAGE_IDS = ["nt", "nn", "tn", "tt"]


@pytest.mark.parametrize("ta,tb", STORAGES, ids=STORAGE_IDS)
@pytest.mark.parametrize("dt", FORMATS8)
@pytest.mark.parametrize("name", ["c1_128", "c1_128_int", "c2_1024", "c4_edge",
                                  "c4_edge_int"])
def test_fp8_small_workloads_full(handle, dt, name, ta, tb):
    """Every storage: A and B stored K-contiguous (K rows of A as M x K, B as
    N x K) or outer-contiguous (read through the 8-bit transposing LDS read)."""
    ops = wl.operands16(W[name], dt, ta=ta, tb=tb)
    out = gu.run16(handle, ops)
    gu.check_full16(ops, out, exact=W[name].dist == "int4", what=f"{name} {dt} {ta}{tb}")


@pytest.mark.parametrize("dt", FORMATS8)
@pytest.mark.parametrize("name", ["c3_4096", "c3_4096_int", "c5_mlp"])
def test_fp8_large_workloads_sampled(handle, dt, name):
    ops = wl.operands16(W[name], dt, tb=True)
    out = gu.run16(handle, ops)
    rows = gu.edge_rows(ops.M, extra=4)[:10]
    cols = [0, 1, 127, 128, 255, 256, ops.N // 2, ops.N - 1]
    gu.check_sampled16(ops, out, rows, cols, exact=W[name].dist == "int4",
                       what=f"{name} {dt}")


@pytest.mark.parametrize("ta,tb", STORAGES, ids=STORAGE_IDS)
@pytest.mark.parametrize("dt", FORMATS8)
def test_fp8_transposed_4096_sampled(handle, dt, ta, tb):
    ops = wl.operands16(W["c3_4096"], dt, ta=ta, tb=tb)
    out = gu.run16(handle, ops)
    gu.check_sampled16(ops, out, [0, 255, 256, 2047, 4095], [0, 256, 4095],
                       npoints=2048, what=f"4096 {dt} ta={ta} tb={tb}")


@pytest.mark.parametrize("dt", FORMATS8)
def test_fp8_tiny_sizes_integer_exact(handle, dt):
    """Sizes 1..70 in every storage: under 16 along an outer-contiguous
    operand the guarded kernel, else the edge or aligned ones."""
    rng = np.random.default_rng(67)
    for case in range(48):
        M, N, K = (int(x) for x in rng.integers(1, 71, size=3))
        ta, tb = STORAGES[case % 4]
        w = wl.Workload("tiny8", 3100 + case, M, N, K, 1.0, 1.0, "int4")
        ops = wl.operands16(w, dt, ta=ta, tb=tb)
        out = gu.run16(handle, ops)
        gu.check_full16(ops, out, exact=True, what=f"tiny {dt} {M}x{N}x{K} {ta}{tb}")


@pytest.mark.parametrize("dt", FORMATS8)
def test_fp8_odd_offsets_and_k_cases(handle, dt):
    """A and B starting at odd byte addresses, odd leading dimensions, K one
    past a K step and K under one step."""
    for i, (M, N, K) in enumerate(((300, 270, 129), (150, 133, 40), (256, 256, 256),
                                   (256, 512, 384))):
        ta, tb = STORAGES[i % 4]
        w = wl.Workload("odd8", 79, M, N, K, 1.25, -0.5, "uniform")
        ops = wl.operands16(w, dt, ta=ta, tb=tb, lda=(M if ta else K) + 3,
                            ldb=(K if tb else N) + 5, ldc=N + 1)
        A, B, C = gu.to_device16(ops)
        t8, u8 = A.dtype, torch.uint8
        A1 = torch.empty(A.numel() + 1, dtype=u8, device=A.device)
        A1[1:] = A.view(u8)
        B1 = torch.empty(B.numel() + 3, dtype=u8, device=B.device)
        B1[3:] = B.view(u8)
        out = gu.run16(handle, ops, dev=(A1.view(t8)[1:], B1.view(t8)[3:], C))
        gu.check_full16(ops, out, what=f"{dt} odd offsets {M}x{N}x{K}")


def test_fp8_storages_agree_bit_for_bit(handle):
    """The same integer problem stored four ways gives the same bits (each
    also matches the oracle exactly)."""
    w = wl.Workload("agree8", 83, 384, 320, 640, 1.5, 0.5, "int4")
    outs = []
    for ta, tb in STORAGES:
        ops = wl.operands16(w, "fp8e4m3", ta=ta, tb=tb)
        out = gu.run16(handle, ops)
        gu.check_full16(ops, out, exact=True, what=f"agree {ta}{tb}")
        outs.append(gu.window(out, ops.M, ops.N, ops.ldc))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("dt", FORMATS8)
@pytest.mark.parametrize("K", [64, 128, 1000])
def test_fp8_wide_range_and_one_signed(handle, dt, K):
    """Inputs spread over seven binades and inputs of one sign: where the
    8-bit instruction's block window loses the most, the results stay inside
    the block allowance of the acceptance."""
    rng = np.random.default_rng([71, K])
    M, N = 192, 160
    for kind in ("wide", "positive"):
        if kind == "wide":
            a = rng.uniform(-1, 1, (M, K)) * 2.0 ** rng.integers(-6, 1, (M, K))
            b = rng.uniform(-1, 1, (N, K)) * 2.0 ** rng.integers(-6, 1, (N, K))
        else:
            a, b = rng.uniform(0, 1, (M, K)), rng.uniform(0, 1, (N, K))
        c = rng.uniform(-1, 1, (M, N)).astype(np.float32)
        ops = wl.Operands16(dt, M, N, K, 0.75, 0.25,
                            wl.place16(wl.round8(a.astype(np.float32), dt), K), K,
                            wl.place16(wl.round8(b.astype(np.float32), dt), K), K,
                            wl.place(c, N), N, False, True)
        out = gu.run16(handle, ops)
        gu.check_full16(ops, out, what=f"{dt} {kind} K={K}")


@pytest.mark.parametrize("dt", [sg.SGEMM_DTYPE_BF16, sg.SGEMM_DTYPE_F16,
                                sg.SGEMM_DTYPE_FP8_E4M3, sg.SGEMM_DTYPE_FP8_E5M2])
def test_mfma_chain_rate_below_peak(dt):
    """The diagnostic chain of each format runs and its rate is plausible:
    above a third of the dense peak and below the peak itself."""
    from fp32_gemm_major_amd import roofline as rf
    peak = rf.PEAK_FP8_FLOPS if dt >= sg.SGEMM_DTYPE_FP8_E4M3 else rf.PEAK_BF16_FLOPS
    tf = sg.mfma_chain_tflops(workgroups=512, iterations=128, reps=2, dtype=dt)
    assert peak / 3e12 < tf < peak / 1e12, tf


def _fp8_family(rng, kind, M, N, K):
    if kind == "wide":
        a = rng.uniform(-1, 1, (M, K)) * 2.0 ** rng.integers(-6, 1, (M, K))
        b = rng.uniform(-1, 1, (N, K)) * 2.0 ** rng.integers(-6, 1, (N, K))
    elif kind == "positive":
        a, b = rng.uniform(0, 1, (M, K)), rng.uniform(0, 1, (N, K))
    elif kind == "uniform":
        a, b = rng.uniform(-1, 1, (M, K)), rng.uniform(-1, 1, (N, K))
    else:
        a, b = rng.normal(0, 0.02, (M, K)), rng.normal(0, 0.02, (N, K))
    return a.astype(np.float32), b.astype(np.float32)


@pytest.mark.parametrize("dt", FORMATS8)
def test_fp8_envelope_measurement(handle, dt):
    """The measurement behind the 8-bit envelope: the worst error of the 8-bit
    product in units of |alpha| * ceil(K/64) * max|a_i.| * max|b_.j| over
    uniform, one-signed, small-normal and seven-binade inputs, K = 64, 128,
    1000 and 4096, for the tile kernels (128 rows: the 32x32x64 instruction)
    and the one-pass small-M kernel (16 rows: the 16x16x128 instruction).
    Printed as a power of two; the allowance is 2^-9."""
    for M in (128, 16):
        _fp8_envelope(handle, dt, M)


def _fp8_envelope(handle, dt, M):
    worst, where, kernel = 0.0, None, None
    for K in (64, 128, 1000, 4096):
        rng = np.random.default_rng([73, K, M])
        N = 96
        for kind in ("wide", "positive", "uniform", "normal"):
            a, b = _fp8_family(rng, kind, M, N, K)
            ops = wl.Operands16(dt, M, N, K, 1.0, 0.0,
                                wl.place16(wl.round8(a, dt), K), K,
                                wl.place16(wl.round8(b, dt), K), K,
                                wl.place(np.full((M, N), np.nan, np.float32), N), N,
                                False, True)
            (kid, _), _ = _plan(handle, ops)
            kernel = sg.sgemm_lowp_kernel_name(kid)
            assert ("_G16x16_" in kernel) == (M <= 16)
            out = gu.run16(handle, ops)
            R, _ = __import__("oracle").gemm_lowp(dt, M, N, K, 1.0, ops.A, K, ops.B, K,
                                                  0.0, None, N, tb=True, with_t=False)
            err = np.abs(gu.window(out, M, N, N).astype(np.float64) - R)
            units = gu.fp8_block_units(ops, np.arange(M)[:, None], np.arange(N)[None, :])
            ratio = float(np.max(err / units))
            if ratio > worst:
                worst, where = ratio, (kind, K)
    print(f"\nfp8 envelope {dt}, {kernel.split('_')[2]} kernels: worst error "
          f"2^{np.log2(worst):.2f} of the block units ({where[0]}, K={where[1]}); "
          f"allowance 2^-9", flush=True)
    assert worst < gu.FP8_BLOCK_ALLOWANCE


@pytest.mark.parametrize("dt", FORMATS8)
def test_fp8_mixed_magnitude_integers(handle, dt):
    """Integer inputs where one block of 64 holds products of very different
    size: a_i0 = +-448 (the largest E4M3 value; E5M2 holds it too) for every
    row, b_0j = +-448 for the first half of the columns and 0 for the rest,
    every other element in [-4, 4].  Every partial sum is an integer below
    2^24, so FP32 accumulation would be exact.  In the first half of the
    columns the first block holds 448*448 beside products as small as 1, which
    the 8-bit instruction's block window may drop; the second half holds
    products of at most 16 and must stay exact.  Checked against the
    envelope; how many outputs stay exact is printed."""
    rng = np.random.default_rng(79)
    M, N, K = 64, 64, 128
    a = rng.integers(-4, 5, (M, K)).astype(np.float32)
    b = rng.integers(-4, 5, (N, K)).astype(np.float32)
    a[:, 0] = 448.0 * rng.choice([-1.0, 1.0], M)
    b[: N // 2, 0] = 448.0 * rng.choice([-1.0, 1.0], N // 2)
    b[N // 2:, 0] = 0.0
    ops = wl.Operands16(dt, M, N, K, 1.0, 0.0, wl.place16(wl.round8(a, dt), K), K,
                        wl.place16(wl.round8(b, dt), K), K,
                        wl.place(np.full((M, N), np.nan, np.float32), N), N, False, True)
    out = gu.run16(handle, ops)
    got = gu.window(out, M, N, N)
    R, _ = __import__("oracle").gemm_lowp(dt, M, N, K, 1.0, ops.A, K, ops.B, K, 0.0,
                                          None, N, tb=True)
    exact = got == __import__("oracle").to_f32(R)
    print(f"\nfp8 mixed magnitudes {dt}: {int(exact[:, : N // 2].sum())} of "
          f"{M * N // 2} outputs with a 448*448 product exact", flush=True)
    assert exact[:, N // 2:].all()  # products of at most 16: exact
    gu.check_full16(ops, out, what=f"{dt} mixed magnitudes")


# ---- split K for products with few rows (a workspace on the handle) ----------

@pytest.fixture(scope="module")
def ws_handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h = sg.Handle()
    yield h
    h.close()


def _plan(h, ops):
    A, B, C = gu.to_device16(ops)
    code = {"bf16": sg.SGEMM_DTYPE_BF16, "f16": sg.SGEMM_DTYPE_F16,
            "fp8e4m3": sg.SGEMM_DTYPE_FP8_E4M3, "fp8e5m2": sg.SGEMM_DTYPE_FP8_E5M2}[ops.dt]
    return sg.sgemm_lowp_plan_handle(h.h, code, int(ops.ta), int(ops.tb), ops.M, ops.N, ops.K,
                                     A.data_ptr(), ops.lda, B.data_ptr(), ops.ldb,
                                     C.data_ptr(), ops.ldc), (A, B, C)


@pytest.mark.parametrize("k", SPLIT_K, ids=[k["name"] for k in SPLIT_K])
def test_split_k_kernels(ws_handle, k):
    """Every split-K kernel, forced, on few-row problems: one row (with A
    stored K x M, the fewest rows the edge kernels take), a ragged row count,
    the most rows it takes; K ragged and long enough for several
    ranges; odd leading dimensions; integers bit-exact, uniform values within
    the bound (the 8-bit envelope for 8-bit formats)."""
    ta, tb = bool(k["transa"]), bool(k["transb"])
    dt = DT_NAME[k["dtype"]]
    ws_handle.set_lowp_kernel(k["id"])
    try:
        # A stored K x M needs M of at least one 16-byte piece (8 or 16 rows)
        piece = 16 if k["dtype"] in (sg.SGEMM_DTYPE_FP8_E4M3, sg.SGEMM_DTYPE_FP8_E5M2) else 8
        for M in ((piece, 37, 64) if ta else (1, 5, 16, 64)):
            for dist in ("int4", "uniform"):
                N, K = 300, 40 * k["bk"] + 19
                w = wl.Workload("lpsk", 9400 + M, M, N, K, 1.5, 0.5, dist)
                ops = wl.operands16(w, dt, ta=ta, tb=tb, lda=(M if ta else K) + 3,
                                    ldb=(K if tb else N) + 5, ldc=N + 2)
                (kid, splits), dev = _plan(ws_handle, ops)
                assert kid == k["id"] and splits >= 2, (kid, splits)
                out = gu.run16(ws_handle, ops, dev=dev)
                gu.check_full16(ops, out, exact=dist == "int4", what=f"{k['name']} M={M} {dist}")
    finally:
        ws_handle.set_lowp_kernel(-1)


@pytest.mark.parametrize("dt", FORMATS + FORMATS8)
@pytest.mark.parametrize("shape", [(1, 4096, 4096), (4, 11008, 4096), (16, 4096, 4096)],
                         ids=["1x4096x4096", "4x11008x4096", "16x4096x4096"])
def test_split_k_plans(ws_handle, dt, shape):
    """Decode-like products (a few rows of A against a weight matrix) on a
    handle with a workspace: when 64x64 tiles fill at most half the CUs
    (N = 4096: 64 tiles), the one-pass kernel with B stored N x K (the 8-bit
    cases) and K split otherwise; one tile per workgroup when they fill more
    (N = 11008: 172 tiles);
    results within the bound (bit-exact on integers), the same bits on
    every run."""
    M, N, K = shape
    tb = dt in FORMATS8
    for dist in ("int4", "uniform"):
        w = wl.Workload("lpskp", 9500 + M, M, N, K, 1.0, 0.5, dist)
        ops = wl.operands16(w, dt, tb=tb)
        (kid, splits), dev = _plan(ws_handle, ops)
        if tb and N == 4096:  # B stored N x K, at most 16 rows: one pass
            assert "_G16x16_" in sg.sgemm_lowp_kernel_name(kid) and splits == 1
        elif N == 4096:
            assert sg.sgemm_lowp_kernel_schedule(kid) == sg.SGEMM_SCHEDULE_SMALL_M
            assert splits >= 2
        else:
            assert sg.sgemm_lowp_kernel_schedule(kid) == sg.SGEMM_SCHEDULE_TILES
            assert splits == 1
        c0 = dev[2].clone()
        out = gu.run16(ws_handle, ops, dev=dev)
        gu.check_full16(ops, out, exact=dist == "int4", what=f"{dt} {shape} {dist}")
        dev[2].copy_(c0)
        again = gu.run16(ws_handle, ops, dev=dev)
        assert np.array_equal(out.view(np.uint32), again.view(np.uint32))


def test_split_k_needs_a_workspace(handle):
    """Without a workspace the planner keeps one tile per workgroup, and a
    forced split-K kernel is refused before anything runs."""
    ops = wl.operands16(wl.Workload("lpnows", 9600, 1, 512, 4096, 1.0, 0.0, "int4"), "bf16")
    (kid, splits), dev = _plan(handle, ops)
    assert sg.sgemm_lowp_kernel_schedule(kid) == sg.SGEMM_SCHEDULE_TILES and splits == 1
    sk = next(k for k in SPLIT_K if k["dtype"] == sg.SGEMM_DTYPE_BF16 and not k["transa"]
              and not k["transb"])
    handle.set_lowp_kernel(sk["id"])
    A, B, C = dev
    c0 = C.clone()
    with pytest.raises(sg.SgemmError) as e:
        handle.gemm_lowp(A, B, C, 1.0, 0.0, M=ops.M, N=ops.N, K=ops.K, lda=ops.lda,
                         ldb=ops.ldb, ldc=ops.ldc)
    assert e.value.status == sg.SGEMM_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.equal(C, c0)


# ---- one pass on the matrix cores: at most 16 rows, B stored N x K -----------

@pytest.mark.parametrize("k", GEMV, ids=[k["name"] for k in GEMV])
def test_gemv_kernels(handle, k):
    """Every one-pass small-M kernel, forced: 1 to 16 rows of A; N not a
    multiple of a workgroup's 16 columns, and N under 16; K over several
    blocks per wave plus a ragged piece, K of one block, and K under one
    16-byte piece; odd leading dimensions.  Integers bit-exact, uniform
    values within the bound (the 8-bit envelope for 8-bit formats)."""
    ta, dt = bool(k["transa"]), DT_NAME[k["dtype"]]
    ue = 16 if k["dtype"] in (sg.SGEMM_DTYPE_FP8_E4M3, sg.SGEMM_DTYPE_FP8_E5M2) else 8
    handle.set_lowp_kernel(k["id"])
    for M in (1, 3, 9, 16):
        for i, (N, K) in enumerate(((300, 37 * k["bk"] + 19), (7, ue - 3), (33, k["bk"]))):
            for dist in ("int4", "uniform"):
                w = wl.Workload("gemv", 9700 + 10 * M + i, M, N, K, 1.5, 0.5, dist)
                ops = wl.operands16(w, dt, ta=ta, tb=True, lda=(M if ta else K) + 3,
                                    ldb=K + 5, ldc=N + 2)
                out = gu.run16(handle, ops)
                gu.check_full16(ops, out, exact=dist == "int4",
                                what=f"{k['name']} {M}x{N}x{K} {dist}")


@pytest.mark.parametrize("dt", FORMATS + FORMATS8)
def test_gemv_unaligned_operands_and_beta_zero(handle, dt):
    """A and B one byte (8-bit) or one element (16-bit) past a 16-byte
    boundary, so every 16-byte piece is unaligned; beta 0 with NaN in C (C is
    not read); K = 0 (C = beta * C)."""
    w = wl.Workload("gemvmis", 9790, 5, 270, 1000, 1.25, -0.5, "uniform")
    ops = wl.operands16(w, dt, tb=True, lda=1003, ldb=1001, ldc=273)
    A, B, C = gu.to_device16(ops)
    u8 = torch.uint8
    off = 1 if dt in FORMATS8 else 2
    na, nb = A.numel() * A.element_size(), B.numel() * B.element_size()
    A1 = torch.empty(na + 2, dtype=u8, device=A.device)
    B1 = torch.empty(nb + 2, dtype=u8, device=B.device)
    A1[off:off + na] = A.view(u8).flatten()
    B1[off:off + nb] = B.view(u8).flatten()
    (kid, _), _ = _plan(handle, ops)
    assert "_G16x16_" in sg.sgemm_lowp_kernel_name(kid)
    out = gu.run16(handle, ops, dev=(A1[off:off + na].view(A.dtype),
                                     B1[off:off + nb].view(B.dtype), C))
    gu.check_full16(ops, out, what=f"{dt} unaligned")
    ops = wl.operands16(W["c2_1024"], dt, M=4, N=100, K=300, tb=True)
    assert np.isnan(ops.C).all()
    out = gu.run16(handle, ops)
    gu.check_full16(ops, out, what=f"{dt} beta 0, NaN C")
    ops = wl.operands16(W["c4_edge"], dt, M=2, N=50, K=0, ldc=53, tb=True)
    out = gu.run16(handle, ops)
    gu.check_full16(ops, out, what=f"{dt} K = 0")


@pytest.mark.parametrize("dt", FORMATS + FORMATS8)
def test_gemv_plans(handle, ws_handle, dt):
    """B stored N x K with at most 16 rows of A runs in one pass when 64x64
    tiles would fill at most half the CUs (N = 4096: 64 tiles) -- except
    that with 16-bit formats, more than four rows and a workspace K is split
    instead; 17 rows, or N = 11008 (172 tiles), do not; the same bits on
    every run."""
    for h in (handle, ws_handle):
        for M, N in ((1, 4096), (4, 4096), (16, 4096), (17, 4096), (4, 11008)):
            w = wl.Workload("gemvp", 9800 + M, M, N, 4096, 1.0, 0.5, "int4")
            ops = wl.operands16(w, dt, tb=True)
            (kid, splits), dev = _plan(h, ops)
            one_pass = M <= 16 and N == 4096 and (
                dt in FORMATS8 or M <= 4 or h is handle)
            assert ("_G16x16_" in sg.sgemm_lowp_kernel_name(kid)) == one_pass
            if not one_pass:
                continue
            assert splits == 1
            c0 = dev[2].clone()
            out = gu.run16(h, ops, dev=dev)
            gu.check_full16(ops, out, exact=True, what=f"{dt} M={M}")
            dev[2].copy_(c0)
            again = gu.run16(h, ops, dev=dev)
            assert np.array_equal(out.view(np.uint32), again.view(np.uint32))


# ---- seeded random problems through the planner ------------------------------

def _random_lowp_problems(seed, count):
    rng = np.random.default_rng(seed)
    picks = []
    for _ in range(count):
        kind = int(rng.integers(0, 4))
        if kind == 0:    # a few rows against a wide B (one-pass, split-K or tiles)
            M = int(rng.integers(1, 20))
            N = int(rng.integers(200, 3000))
            K = int(rng.integers(100, 3000))
        elif kind == 1:  # tile multiples give or take a little
            M = int(rng.choice([64, 128, 256])) * int(rng.integers(1, 5)) + int(rng.integers(-3, 4))
            N = int(rng.choice([64, 128, 256])) * int(rng.integers(1, 5)) + int(rng.integers(-3, 4))
            K = int(rng.choice([64, 128])) * int(rng.integers(1, 10)) + int(rng.integers(-2, 3))
        elif kind == 2:  # few tiles, deep K
            M = int(rng.integers(17, 200))
            N = int(rng.integers(17, 200))
            K = int(rng.integers(1000, 4000))
        else:            # anything up to mid sizes
            M, N, K = (int(x) for x in rng.integers(1, 700, size=3))
        M, N, K = max(M, 1), max(N, 1), max(K, 1)
        ta, tb = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
        alpha = float(rng.choice([1.0, -1.5, 0.5]))
        beta = float(rng.choice([0.0, 1.0, -0.5]))
        pads = [int(x) for x in rng.integers(0, 5, size=3)]
        picks.append((M, N, K, ta, tb, alpha, beta, pads))
    return picks


@pytest.mark.parametrize("dt", FORMATS + FORMATS8)
def test_random_problems_integer_exact(ws_handle, dt):
    """12 seeded random problems per format through sgemm_run_lowp's planner
    on a handle with a workspace (so the one-pass and split-K small-M kernels
    are candidates): random storage, sizes, strides, alpha and beta;
    bit-exact on integer inputs, the padding of C untouched."""
    seed = {"bf16": 0, "f16": 1, "fp8e4m3": 2, "fp8e5m2": 3}[dt]
    for i, (M, N, K, ta, tb, alpha, beta, pads) in enumerate(
            _random_lowp_problems(9900 + seed, 12)):
        w = wl.Workload("lprand", 9910 + 16 * seed + i, M, N, K, alpha, beta, "int4",
                        "nan" if beta == 0.0 else "dist")
        ops = wl.operands16(w, dt, ta=ta, tb=tb, lda=(M if ta else K) + pads[0],
                            ldb=(K if tb else N) + pads[1], ldc=N + pads[2])
        (kid, splits), dev = _plan(ws_handle, ops)
        what = (f"{dt} {M}x{N}x{K} ta={ta} tb={tb} a={alpha} b={beta} pads={pads} "
                f"kernel={sg.sgemm_lowp_kernel_name(kid)} splits={splits}")
        print(what, flush=True)
        out = gu.run16(ws_handle, ops, dev=dev)
        gu.check_full16(ops, out, exact=True, what=what)
