"""Host-side checks of the 16-bit and 8-bit products' C ABI (no GPU, nothing
launched)."""
import pytest

import fp32_gemm_major_amd as sg

BF16, F16 = sg.SGEMM_DTYPE_BF16, sg.SGEMM_DTYPE_F16
E4M3, E5M2 = sg.SGEMM_DTYPE_FP8_E4M3, sg.SGEMM_DTYPE_FP8_E5M2


def test_validate_lowp():
    v = sg.sgemm_validate_lowp
    A, B, C = 0x10000, 0x20000, 0x40000  # disjoint fake addresses (never touched)
    ok = sg.SGEMM_OK
    assert v(BF16, 0, 0, 4, 5, 6, A, 6, B, 5, 0.0, C, 5) == ok
    assert v(F16, 1, 1, 4, 5, 6, A, 4, B, 6, 0.0, C, 5) == ok
    assert v(0, 0, 0, 4, 5, 6, A, 6, B, 5, 0.0, C, 5) == sg.SGEMM_ERR_VALUE
    assert v(5, 0, 0, 4, 5, 6, A, 6, B, 5, 0.0, C, 5) == sg.SGEMM_ERR_VALUE
    # 8-bit formats: 1-byte elements, no alignment, windows in bytes
    assert v(E4M3, 0, 1, 4, 5, 6, A + 1, 6, B + 3, 6, 0.0, C, 5) == ok
    assert v(E5M2, 0, 1, 4, 5, 6, A, 6, B, 6, 0.0, A + 23, 5) == sg.SGEMM_ERR_ALIAS
    assert v(E5M2, 0, 1, 4, 5, 6, A, 6, B, 6, 0.0, A + 24, 5) == ok
    assert v(BF16, 2, 0, 4, 5, 6, A, 6, B, 5, 0.0, C, 5) == sg.SGEMM_ERR_VALUE
    assert v(BF16, 0, 0, -1, 5, 6, A, 6, B, 5, 0.0, C, 5) == sg.SGEMM_ERR_SIZE
    assert v(BF16, 0, 0, 4, 5, 6, A, 5, B, 5, 0.0, C, 5) == sg.SGEMM_ERR_LD
    assert v(BF16, 1, 0, 4, 5, 6, A, 3, B, 5, 0.0, C, 5) == sg.SGEMM_ERR_LD  # K x M: lda >= M
    assert v(BF16, 0, 1, 4, 5, 6, A, 6, B, 5, 0.0, C, 5) == sg.SGEMM_ERR_LD  # N x K: ldb >= K
    assert v(BF16, 0, 0, 4, 5, 6, A, 6, B, 5, 0.0, C, 4) == sg.SGEMM_ERR_LD
    assert v(BF16, 0, 0, 4, 5, 6, None, 6, B, 5, 0.0, C, 5) == sg.SGEMM_ERR_NULL
    assert v(BF16, 0, 0, 4, 5, 6, A, 6, B, 5, 0.0, None, 5) == sg.SGEMM_ERR_NULL
    assert v(BF16, 0, 0, 4, 5, 0, None, 1, None, 5, 1.0, C, 5) == ok  # K == 0
    assert v(BF16, 0, 0, 0, 5, 6, None, 6, None, 5, 1.0, None, 5) == ok  # empty
    # 2-byte elements must be 2-byte aligned
    assert v(BF16, 0, 0, 4, 5, 6, A + 1, 6, B, 5, 0.0, C, 5) == sg.SGEMM_ERR_VALUE
    assert v(F16, 0, 0, 4, 5, 6, A, 6, B + 3, 5, 0.0, C, 5) == sg.SGEMM_ERR_VALUE
    assert v(F16, 0, 0, 4, 5, 6, A + 2, 6, B + 6, 5, 0.0, C, 5) == ok
    # overlap is measured in bytes: A spans 4*6 two-byte elements
    assert v(BF16, 0, 0, 4, 5, 6, A, 6, B, 5, 0.0, A + 46, 5) == sg.SGEMM_ERR_ALIAS
    assert v(BF16, 0, 0, 4, 5, 6, A, 6, B, 5, 0.0, A + 48, 5) == ok
    assert v(BF16, 0, 0, 4, 5, 6, A, 6, B, 5, 0.0, B + 2 * 29, 5) == sg.SGEMM_ERR_ALIAS
    assert v(BF16, 0, 0, 4, 5, 6, A, 6, B, 5, 0.0, B + 2 * 30, 5) == ok


def test_null_handle():
    lib = sg.library()
    assert lib.sgemm_run_lowp(None, BF16, 0, 0, 4, 4, 4, 1.0, 16, 4, 16, 4, 0.0, 4096, 4,
                              None) == sg.SGEMM_ERR_HANDLE
    assert lib.sgemm_set_lowp_kernel(None, 0) == sg.SGEMM_ERR_HANDLE


def test_kernel_table():
    t = sg.lowp_kernel_table()
    names = [k["name"] for k in t]
    assert len(set(names)) == len(names) == sg.sgemm_lowp_num_kernels()
    combos = {(k["dtype"], k["transa"], k["transb"], k["bm"], k["mode"]) for k in t}
    for dt in (BF16, F16, E4M3, E5M2):
        for ta in (0, 1):
            for tb in (0, 1):
                for bm in (64, 128, 256):
                    assert (dt, ta, tb, bm, sg.SGEMM_MODE_ALIGNED) in combos
                for bm in (64, 128):
                    assert (dt, ta, tb, bm, sg.SGEMM_MODE_EDGE) in combos
                assert (dt, ta, tb, 64, sg.SGEMM_MODE_GUARDED) in combos
    gemv = [k for k in t if "_G16x16_" in k["name"]]
    for k in t:
        assert ("bf16" in k["name"]) == (k["dtype"] == BF16)
        tag = {(0, 0): "", (1, 0): "tn_", (0, 1): "nt_", (1, 1): "tt_"}[(k["transa"], k["transb"])]
        assert f"x{k['bn']}_{tag}" in k["name"]
        if k in gemv:
            continue
        assert k["threads"] == 256
        assert k["bk"] == (128 if k["dtype"] >= E4M3 else 64)
        assert k["bm"] == k["bn"]
    # the one-pass small-M kernels: every format, A in either storage, B
    # stored N x K; 16 rows of A and 16 columns per workgroup of 8 waves, K
    # in blocks of one 16 x 16 MFMA (32 k of a 16-bit format, 128 of an 8-bit
    # one)
    assert sorted((k["dtype"], k["transa"]) for k in gemv) == sorted(
        (dt, ta) for dt in (BF16, F16, E4M3, E5M2) for ta in (0, 1))
    for k in gemv:
        assert k["transb"] == 1 and (k["bm"], k["bn"], k["threads"]) == (16, 16, 512)
        assert k["bk"] == (128 if k["dtype"] >= E4M3 else 32)
        assert k["schedule"] == sg.SGEMM_SCHEDULE_SMALL_M and k["name"].endswith("_small")
    assert sg.sgemm_lowp_kernel_name(-1) is None
    assert sg.sgemm_lowp_kernel_name(len(t)) is None
    with pytest.raises(sg.SgemmError):
        sg.sgemm_lowp_kernel_info(len(t))


def _pick(dt, M, N, K, lda=None, ldb=None, ta=0, tb=0, A=1 << 20, B=1 << 33,
          C=1 << 38):
    lda = lda or (M if ta else K)
    ldb = ldb or (K if tb else N)
    kid = sg.sgemm_lowp_select_kernel(dt, ta, tb, M, N, K, A, lda, B, ldb, C, N)
    return sg.sgemm_lowp_kernel_info(kid) if kid >= 0 else kid


@pytest.mark.parametrize("dt", [BF16, F16])
@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_select(dt, ta, tb):
    A, E, G = sg.SGEMM_MODE_ALIGNED, sg.SGEMM_MODE_EDGE, sg.SGEMM_MODE_GUARDED
    k = _pick(dt, 4096, 4096, 4096, ta=ta, tb=tb)
    assert (k["bm"], k["mode"], k["dtype"]) == (256, A, dt)
    assert (k["transa"], k["transb"]) == (ta, tb)
    k = _pick(dt, 2048, 2048, 1024, ta=ta, tb=tb)  # 64 tiles of 256, 256 of 128
    assert (k["bm"], k["mode"]) == (128, A)
    k = _pick(dt, 1024, 1024, 1024, ta=ta, tb=tb)  # 64 tiles of 128: use 64
    assert (k["bm"], k["mode"]) == (64, A)
    # 144 tiles of 256 (one partial round) against 576 of 128 (three rounds)
    k = _pick(dt, 3072, 3072, 1024, ta=ta, tb=tb)
    assert (k["bm"], k["mode"]) == (256, A)
    # 128 tiles of 256 against 512 of 128: two rounds of the smaller tile
    k = _pick(dt, 2048, 4096, 1024, ta=ta, tb=tb)
    assert (k["bm"], k["mode"]) == (128, A)
    # not tile multiples: the 128x128 edge kernel stands in for 256x256
    k = _pick(dt, 3000, 3000, 1000, ta=ta, tb=tb)
    assert (k["bm"], k["mode"]) == (128, E)
    k = _pick(dt, 1000, 1500, 777, ta=ta, tb=tb)
    assert (k["bm"], k["mode"]) == (64, E)
    k = _pick(dt, 4100, 4100, 4100, ta=ta, tb=tb)  # edge kernels stop at 128
    assert (k["bm"], k["mode"]) == (128, E)
    # multiples of 128 but not of 256, with the 256x256 tile preferred (three
    # or more rounds of 128x128 tiles): the aligned 128x128 instance, not an
    # edge one
    k = _pick(dt, 3200, 3200, 1024, ta=ta, tb=tb)
    assert (k["bm"], k["mode"]) == (128, A)
    # direct loads take any 2-byte alignment: odd leading dimensions and a
    # base off 16 bytes stay aligned
    k = _pick(dt, 4096, 4096, 4096, lda=4099, ta=ta, tb=tb)
    assert (k["bm"], k["mode"]) == (256, A)
    k = _pick(dt, 4096, 4096, 4096, A=(1 << 20) + 2, ta=ta, tb=tb)
    assert k["mode"] == A
    assert _pick(dt, 4096, 4096, 4096, A=(1 << 20) + 1) == sg.SGEMM_ERR_VALUE
    # an extent under 8 along an outer-contiguous operand's pieces (seven
    # rows of A with B stored N x K: the one-pass small-M kernel instead)
    k = _pick(dt, 7 if ta else 300, 300 if ta else (300 if tb else 7), 100, ta=ta, tb=tb)
    if ta and tb:
        assert "_G16x16_" in k["name"]
    elif ta or not tb:
        assert (k["bm"], k["mode"]) == (64, G)
    else:
        assert k["mode"] == E


def test_huge_strides_go_to_the_guarded_kernel():
    """An operand whose tile spans more than 4 GiB in one K step cannot use
    the 32-bit lane offsets of the direct loads."""
    # 255 rows of lda 2^24 + 8 pass 4 GiB, 127 rows (the 128x128 tiles) do not:
    # the aligned 128x128 instance takes it
    k = _pick(BF16, 4096, 4096, 4096, lda=(1 << 24) + 8)
    assert (k["bm"], k["mode"]) == (128, sg.SGEMM_MODE_ALIGNED)
    k = _pick(BF16, 4096, 4096, 4096, lda=(1 << 25) + 8, B=1 << 42, C=1 << 44)
    assert k["mode"] == sg.SGEMM_MODE_GUARDED
    # stored K x M, one K step of a tile spans 63 rows of A
    k = _pick(BF16, 4096, 4096, 4096, lda=(1 << 24) + 8, ta=1)
    assert k["mode"] == sg.SGEMM_MODE_ALIGNED
    k = _pick(BF16, 4096, 4096, 4096, lda=(1 << 26) + 8, ta=1, B=1 << 42, C=1 << 44)
    assert k["mode"] == sg.SGEMM_MODE_GUARDED


@pytest.mark.parametrize("dt", [E4M3, E5M2])
def test_select_fp8(dt):
    A, E = sg.SGEMM_MODE_ALIGNED, sg.SGEMM_MODE_EDGE
    k = _pick(dt, 4096, 4096, 4096, tb=1)
    assert (k["bm"], k["mode"], k["dtype"], k["bk"]) == (256, A, dt, 128)
    k = _pick(dt, 4096, 4096, 4160, tb=1)   # K not a multiple of 128
    assert (k["bm"], k["mode"]) == (128, E)
    k = _pick(dt, 1024, 1024, 1024, tb=1, A=(1 << 20) + 1, B=(1 << 33) + 3)
    assert (k["bm"], k["mode"]) == (64, A)
    # every storage: A or B stored outer-contiguous (read by transposing reads)
    for ta, tb in ((0, 0), (1, 0), (1, 1)):
        k = _pick(dt, 4096, 4096, 4096, ta=ta, tb=tb)
        assert (k["bm"], k["mode"], k["transa"], k["transb"]) == (256, A, ta, tb)
        k = _pick(dt, 1000, 1500, 777, ta=ta, tb=tb)
        assert (k["bm"], k["mode"]) == (64, E)
    # an outer-contiguous 8-bit piece is 16 elements: 15 columns of B stored
    # K x N go to the guarded kernel, 16 to the edge one
    assert _pick(dt, 300, 15, 200)["mode"] == sg.SGEMM_MODE_GUARDED
    assert _pick(dt, 300, 16, 200)["mode"] == E
    assert _pick(dt, 15, 300, 200, ta=1)["mode"] == sg.SGEMM_MODE_GUARDED
    assert _pick(dt, 16, 300, 200, ta=1)["mode"] == E
    assert _pick(dt, 17, 300, 200, ta=1, tb=1)["mode"] == E


@pytest.mark.parametrize("dt", [BF16, F16, E4M3, E5M2])
@pytest.mark.parametrize("ta", [0, 1])
def test_select_small_m_one_pass(dt, ta):
    """At most 16 rows of A against B stored N x K, with 64x64 tiles for at
    most half the CUs: the one-pass matrix-core kernel, also without a
    workspace; not with 17 rows, with B stored K x N, or with 172 tiles."""
    for M, N, K in ((1, 4096, 4096), (16, 4096, 4096), (3, 300, 5), (1, 8192, 1000)):
        k = _pick(dt, M, N, K, ta=ta, tb=1)
        assert "_G16x16_" in k["name"] and k["schedule"] == sg.SGEMM_SCHEDULE_SMALL_M
        assert (k["dtype"], k["transa"], k["transb"]) == (dt, ta, 1)
    for M, N, K, tb in ((17, 4096, 4096, 1), (1, 4096, 4096, 0), (4, 11008, 4096, 1),
                        (1, 8256, 4096, 1)):
        k = _pick(dt, M, N, K, ta=ta, tb=tb)
        assert k["schedule"] == sg.SGEMM_SCHEDULE_TILES, (M, N, K, tb, k["name"])
    # K within 1024 of 2^31: the one-pass kernel's 32-bit k would pass it
    big = (1 << 31) - 1000
    k = _pick(dt, 1, 64, big, ta=ta, tb=1, A=1 << 20, B=1 << 40, C=1 << 46)
    assert isinstance(k, int) or "_G16x16_" not in k["name"]
    k = _pick(dt, 1, 64, big - 100, ta=ta, tb=1, A=1 << 20, B=1 << 40, C=1 << 46)
    assert not isinstance(k, int) and "_G16x16_" in k["name"]


def test_diag_chain_argument_errors():
    """Argument checks of the low-precision MFMA chain come before any HIP call."""
    f = sg.library().sgemm_diag_mfma_chain_lowp  # raw status codes
    assert f(0, 1, 1, 0x1000, 0) == sg.SGEMM_ERR_VALUE
    assert f(E5M2 + 1, 1, 1, 0x1000, 0) == sg.SGEMM_ERR_VALUE
    for dt in (BF16, F16, E4M3, E5M2):
        assert f(dt, 0, 1, 0x1000, 0) == sg.SGEMM_ERR_SIZE
        assert f(dt, 1, -1, 0x1000, 0) == sg.SGEMM_ERR_SIZE
        assert f(dt, 1, 1, 0, 0) == sg.SGEMM_ERR_NULL
