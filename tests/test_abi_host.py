"""Host-side checks of the C ABI library (no GPU needed, no kernel launched)."""
import ctypes
import os
import re

import numpy as np
import pytest

import fp32_gemm_major_amd as sg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgemm.h")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sgemm_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = sg.library()
    names = declared_functions()
    assert "sgemm_create" in names and "sgemm_run" in names and "sgemm_destroy" in names
    for name in names:
        assert hasattr(lib, name), f"{name} declared in include/sgemm.h but not exported"
    assert set(names) == set(sg.EXPORTED)


def test_null_handle_and_destroy():
    lib = sg.library()
    assert lib.sgemm_destroy(None) == 0
    assert lib.sgemm_run(None, 4, 4, 4, 1.0, 16, 4, 16, 4, 0.0, 4096, 4, None) == sg.SGEMM_ERR_HANDLE
    assert lib.sgemm_set_variant(None, 1) == sg.SGEMM_ERR_HANDLE
    assert lib.sgemm_set_kernel(None, 0) == sg.SGEMM_ERR_HANDLE
    assert lib.sgemm_create(None) == sg.SGEMM_ERR_HANDLE
    assert lib.sgemm_diag_run_clocked(None, 0, 0, 4, 4, 4, 1.0, 16, 4, 16, 4, 0.0, 4096, 4,
                                      8192, 1, None) == sg.SGEMM_ERR_HANDLE
    assert lib.sgemm_diag_wall_clock_khz(None) == sg.SGEMM_ERR_NULL
    assert lib.sgemm_run_ex_noalloc(None, 0, 0, 4, 4, 4, 1.0, 16, 4, 16, 4, 0.0, 4096, 4,
                                    None) == sg.SGEMM_ERR_HANDLE


def test_validate():
    v = sg.sgemm_validate
    A, B, C = 0x10000, 0x20000, 0x40000  # disjoint fake addresses (never touched)
    assert v(4, 5, 6, A, 6, B, 5, 0.0, C, 5) == sg.SGEMM_OK
    assert v(-1, 5, 6, A, 6, B, 5, 0.0, C, 5) == sg.SGEMM_ERR_SIZE
    assert v(4, -5, 6, A, 6, B, 5, 0.0, C, 5) == sg.SGEMM_ERR_SIZE
    assert v(4, 5, -6, A, 6, B, 5, 0.0, C, 5) == sg.SGEMM_ERR_SIZE
    assert v(4, 5, 6, A, 5, B, 5, 0.0, C, 5) == sg.SGEMM_ERR_LD
    assert v(4, 5, 6, A, 6, B, 4, 0.0, C, 5) == sg.SGEMM_ERR_LD
    assert v(4, 5, 6, A, 6, B, 5, 0.0, C, 4) == sg.SGEMM_ERR_LD
    assert v(4, 5, 0, None, 1, None, 5, 1.0, C, 5) == sg.SGEMM_OK  # K == 0: A, B unused
    assert v(4, 5, 0, None, 0, None, 5, 1.0, C, 5) == sg.SGEMM_ERR_LD  # lda >= 1
    assert v(0, 5, 6, None, 6, None, 5, 1.0, None, 5) == sg.SGEMM_OK  # empty: nothing touched
    assert v(4, 0, 6, None, 6, None, 1, 1.0, None, 1) == sg.SGEMM_OK
    assert v(4, 5, 6, None, 6, B, 5, 0.0, C, 5) == sg.SGEMM_ERR_NULL
    assert v(4, 5, 6, A, 6, None, 5, 0.0, C, 5) == sg.SGEMM_ERR_NULL
    assert v(4, 5, 6, A, 6, B, 5, 0.0, None, 5) == sg.SGEMM_ERR_NULL
    # C overlapping A or B
    assert v(4, 5, 6, A, 6, B, 5, 0.0, A + 4, 5) == sg.SGEMM_ERR_ALIAS
    assert v(4, 5, 6, A, 6, B, 5, 0.0, B + 4 * 19, 5) == sg.SGEMM_ERR_ALIAS
    # adjacent but not overlapping: C starts right after A's last element
    assert v(4, 5, 6, A, 6, B, 5, 0.0, A + 4 * 24, 5) == sg.SGEMM_OK


def test_validate_transposed():
    v = sg.sgemm_validate_ex
    A, B, C = 0x10000, 0x20000, 0x40000
    N_, T_ = sg.SGEMM_OP_N, sg.SGEMM_OP_T
    # op(A) = A^T: A stored K x M, lda >= M
    assert v(T_, N_, 4, 5, 6, A, 4, B, 5, 0.0, C, 5) == sg.SGEMM_OK
    assert v(T_, N_, 4, 5, 6, A, 3, B, 5, 0.0, C, 5) == sg.SGEMM_ERR_LD
    assert v(T_, N_, 8, 5, 2, A, 8, B, 5, 0.0, C, 5) == sg.SGEMM_OK  # lda < K is fine
    # op(B) = B^T: B stored N x K, ldb >= K
    assert v(N_, T_, 4, 5, 6, A, 6, B, 6, 0.0, C, 5) == sg.SGEMM_OK
    assert v(N_, T_, 4, 5, 6, A, 6, B, 5, 0.0, C, 5) == sg.SGEMM_ERR_LD
    assert v(2, N_, 4, 5, 6, A, 6, B, 5, 0.0, C, 5) == sg.SGEMM_ERR_VALUE
    assert v(N_, -1, 4, 5, 6, A, 6, B, 5, 0.0, C, 5) == sg.SGEMM_ERR_VALUE
    # alias windows follow the stored shapes: A^T is 6 rows of lda 4
    assert v(T_, N_, 4, 5, 6, A, 4, B, 5, 0.0, A + 4 * 20, 5) == sg.SGEMM_ERR_ALIAS
    assert v(T_, N_, 4, 5, 6, A, 4, B, 5, 0.0, A + 4 * 24, 5) == sg.SGEMM_OK
    # the plain entry points are the N/N case
    assert v(N_, N_, 4, 5, 6, A, 6, B, 5, 0.0, C, 5) == sg.sgemm_validate(
        4, 5, 6, A, 6, B, 5, 0.0, C, 5)


def test_plan_transposed():
    A, B, C = 0x10000000, 0x20000000, 0x40000000
    for ta in (0, 1):
        for tb in (0, 1):
            p = sg.sgemm_plan(0, 4096, 4096, 4096, A, 4096, B, 4096, C, 4096,
                              transa=ta, transb=tb)
            info = sg.sgemm_kernel_info(p[0][0])
            assert len(p) == 1 and (info["transa"], info["transb"]) == (ta, tb)
            assert info["mode"] == sg.SGEMM_MODE_ALIGNED and info["bm"] == 256
    with pytest.raises(sg.SgemmError) as e:
        sg.sgemm_plan(sg.SGEMM_VARIANT_VALU, 64, 64, 64, A, 64, B, 64, C, 64, transa=1)
    assert e.value.status == sg.SGEMM_ERR_UNSUPPORTED


def test_aligned_kernels_need_whole_stages_of_k():
    """An aligned kernel is chosen only when K is a multiple of its stage."""
    A, B, C = 0x10000000, 0x20000000, 0x40000000
    for K in (16, 48, 80, 1040, 1024, 4096):
        for M, N in ((256, 192), (1024, 1024), (4096, 4096)):
            for kid, _, _ in sg.sgemm_plan(0, M, N, K, A, K, B, N, C, N):
                info = sg.sgemm_kernel_info(kid)
                if info["mode"] == sg.SGEMM_MODE_ALIGNED:
                    assert K % info["bk"] == 0 and M % info["bm"] == 0, (M, N, K, info)


def test_status_strings():
    for code in range(-10, 1):
        s = sg.sgemm_status_string(code)
        assert s and s != "unknown status"
    assert sg.sgemm_status_string(-100) == "unknown status"


def test_kernel_table():
    table = sg.kernel_table()
    assert len(table) == sg.sgemm_num_kernels() >= 4
    assert sg.sgemm_kernel_name(-1) is None and sg.sgemm_kernel_name(len(table)) is None
    variants = {k["variant"] for k in table}
    assert variants == {sg.SGEMM_VARIANT_MFMA, sg.SGEMM_VARIANT_VALU}
    for k in table:
        assert k["bm"] > 0 and k["bn"] > 0 and k["bk"] > 0 and k["threads"] % 64 == 0
    # every MFMA tile shape has an aligned, an edge and a guarded instance for
    # each storage; the VALU shape an aligned and a guarded one; the small-M
    # kernels one edge instance per storage: on the vector ALUs 1, 2, 4 and 8
    # rows (one pass, 32 columns per workgroup) and 4, 8 and 16 rows (K split,
    # 256 columns) with B as stored, 1, 2, 4 and 8 rows with B transposed
    # (one pass, 8 columns per workgroup up to 2 rows, else 4); on the matrix
    # cores (K split) one tile row, 32 with A as stored, 64 with A transposed
    skinny = [k for k in table if k["schedule"] == sg.SGEMM_SCHEDULE_SMALL_M]
    for k in skinny:
        if k["variant"] == sg.SGEMM_VARIANT_VALU and k["transb"]:
            assert k["bn"] == (8 if k["bm"] <= 2 else 4) and k["threads"] == 512, k
        elif k["variant"] == sg.SGEMM_VARIANT_VALU:
            assert (k["bn"], k["threads"]) == ((32, 1024) if "x32_" in k["name"] else (256, 512)), k
            assert ("x32_" in k["name"]) == (k["bk"] == 32), k
    assert sorted((k["bm"], k["transa"], k["transb"], k["mode"], k["variant"]) for k in skinny) == \
        sorted([(m, a, b, sg.SGEMM_MODE_EDGE, sg.SGEMM_VARIANT_VALU)
                for a in (0, 1) for b in (0, 1)
                for m in ((1, 2, 4, 8) if b else (1, 2, 4, 8, 4, 8, 16))] +
               [(64 if a else 32, a, b, sg.SGEMM_MODE_EDGE, sg.SGEMM_VARIANT_MFMA)
                for a in (0, 1) for b in (0, 1)])
    shapes = {(k["variant"], k["bm"], k["bn"], k["bk"]) for k in table
              if k["schedule"] != sg.SGEMM_SCHEDULE_SMALL_M}
    for s in shapes:
        inst = {(k["transa"], k["transb"], k["mode"]) for k in table
                if (k["variant"], k["bm"], k["bn"], k["bk"]) == s
                and k["schedule"] != sg.SGEMM_SCHEDULE_SMALL_M}
        if s[0] == sg.SGEMM_VARIANT_VALU:
            want = {(0, 0, sg.SGEMM_MODE_ALIGNED), (0, 0, sg.SGEMM_MODE_GUARDED)}
        else:
            # tiles of fewer than 64 rows take only A stored M x K
            want = {(a, b, m) for a in ((0, 1) if s[1] >= 64 else (0,)) for b in (0, 1)
                    for m in (sg.SGEMM_MODE_ALIGNED, sg.SGEMM_MODE_EDGE,
                              sg.SGEMM_MODE_GUARDED)}
        assert inst == want, s


def test_select_kernel():
    sel = sg.sgemm_select_kernel
    A, B, C = 0x10000, 0x20000, 0x40000
    for variant in (sg.SGEMM_VARIANT_AUTO, sg.SGEMM_VARIANT_MFMA, sg.SGEMM_VARIANT_VALU):
        want = sg.SGEMM_VARIANT_MFMA if variant != sg.SGEMM_VARIANT_VALU else variant
        k = sg.sgemm_kernel_info(sel(variant, 4096, 4096, 4096, A, 4096, B, 4096, C, 4096))
        assert k["variant"] == want and k["mode"] == sg.SGEMM_MODE_ALIGNED
        assert 4096 % k["bm"] == 0 and 4096 % k["bn"] == 0
        mfma = want == sg.SGEMM_VARIANT_MFMA
        # ragged sizes, rows of A only 4-byte aligned: the MFMA edge instance
        k = sg.sgemm_kernel_info(sel(variant, 1000, 1500, 777, A, 777, B, 1500, C, 1500))
        assert k["mode"] == (sg.SGEMM_MODE_EDGE if mfma else sg.SGEMM_MODE_GUARDED)
        # N not a multiple of 4 with B as stored: still the edge instance
        k = sg.sgemm_kernel_info(sel(variant, 1000, 1501, 777, A, 777, B, 1501, C, 1501))
        assert k["mode"] == (sg.SGEMM_MODE_EDGE if mfma else sg.SGEMM_MODE_GUARDED)
        # fewer than 4 columns with B as stored: only the guarded instance
        k = sg.sgemm_kernel_info(sel(variant, 1000, 3, 777, A, 777, B, 3, C, 3))
        assert k["mode"] == sg.SGEMM_MODE_GUARDED
        # a base pointer off 16-byte alignment: MFMA direct loads take it
        k = sg.sgemm_kernel_info(sel(variant, 1024, 1024, 1024, A + 4, 1024, B, 1024, C, 1024))
        assert k["mode"] == (sg.SGEMM_MODE_ALIGNED if mfma else sg.SGEMM_MODE_GUARDED)
    assert sel(7, 64, 64, 64, A, 64, B, 64, C, 64) == sg.SGEMM_ERR_VALUE
    # tile shapes the cost model picks for the measured workloads: 4096^3 on a
    # large tile filling whole rounds, and 32 x 64 for the small and ragged
    # problems (1000 x 1500: 768 tiles, three per CU, where 64 x 64 leaves
    # half the CUs with two tiles and half with one; 4096 x 11008 is covered
    # by the launch-plan test)
    def shape(M, N, K):
        k = sg.sgemm_kernel_info(sel(0, M, N, K, A, K, B, N, C, N))
        return k["bm"], k["bn"]
    bm, bn = shape(4096, 4096, 4096)
    assert bm * bn >= 128 * 128 and (4096 // bm) * (4096 // bn) % 256 == 0
    assert shape(1024, 1024, 1024) == (32, 64)
    assert shape(128, 128, 128) == (32, 64)
    assert shape(1000, 1500, 777) == (32, 64)


def test_plan_splits_only_when_rounds_are_ragged():
    A, B, C = 0x10000000, 0x20000000, 0x40000000
    plan = lambda M, N, K: sg.sgemm_plan(0, M, N, K, A, K, B, N, C, N)
    # 4096^3 fills whole rounds of any tile: one launch
    assert len(plan(4096, 4096, 4096)) == 1
    for M, N, K in [(128, 128, 128), (1024, 1024, 1024), (1000, 1500, 777)]:
        assert len(plan(M, N, K)) == 1
    # 4096 x 11008: whole rounds of a large tile, then the remaining columns
    p = plan(4096, 11008, 4096)
    assert len(p) == 2
    (k0, c0, n0), (k1, c1, n1) = p
    i0, i1 = sg.sgemm_kernel_info(k0), sg.sgemm_kernel_info(k1)
    assert c0 == 0 and c1 == n0 and n0 + n1 == 11008
    assert n0 % i0["bn"] == 0 and (4096 // i0["bm"]) * (n0 // i0["bn"]) % 256 == 0
    assert i0["mode"] == sg.SGEMM_MODE_ALIGNED
    assert i1["mode"] == (sg.SGEMM_MODE_ALIGNED if n1 % i1["bn"] == 0 else sg.SGEMM_MODE_EDGE)
    assert i0["bm"] * i0["bn"] >= i1["bm"] * i1["bn"]
    # the first launch's kernel is what sgemm_select_kernel reports
    assert sg.sgemm_select_kernel(0, 4096, 11008, 4096, A, 4096, B, 11008, C, 11008) == k0
    # tiny K: a second launch never pays
    assert len(plan(4096, 11008, 16)) == 1


@pytest.mark.parametrize("tiles_m,tiles_n", [(1, 1), (16, 16), (16, 43), (7, 9), (3, 1),
                                             (1, 5), (8, 8), (13, 86), (32, 32)])
def test_tile_map_is_a_bijection(tiles_m, tiles_n):
    nwg = tiles_m * tiles_n
    seen = set()
    for wg in range(nwg):
        tm, tn = sg.sgemm_tile_coords(wg, nwg, tiles_m, tiles_n)
        assert 0 <= tm < tiles_m and 0 <= tn < tiles_n
        seen.add((tm, tn))
    assert len(seen) == nwg


@pytest.mark.parametrize("tiles,rows,cols", [(16, 4, 8), (32, 8, 16)])
def test_tile_map_groups_each_xcd(tiles, rows, cols):
    # each XCD (workgroup ids congruent mod 8) owns a near-square block of tiles:
    # 16 x 16 tiles -> 4 x 8 per XCD; 32 x 32 tiles (4096^3 on 128 x 128) -> 8 x 16
    nwg = tiles * tiles
    for x in range(8):
        coords = [sg.sgemm_tile_coords(wg, nwg, tiles, tiles) for wg in range(x, nwg, 8)]
        assert len({c[0] for c in coords}) == rows
        assert len({c[1] for c in coords}) == cols


def test_create_without_gpu_fails_cleanly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    h = ctypes.c_void_p()
    rc = sg.library().sgemm_create(ctypes.byref(h))
    assert rc in (sg.SGEMM_ERR_DEVICE, sg.SGEMM_ERR_HIP) and not h.value


def test_huge_strides_go_to_the_guarded_instance():
    """Direct loads address a tile with 32-bit lane offsets: when one K step of
    every MFMA tile spans 4 GiB or more, only the guarded instance fits."""
    A, B, C = 0x10000000, 0x20000000, 0x40000000
    M, N, K = 70, 160, 40
    small = sg.sgemm_kernel_info(sg.sgemm_select_kernel(0, M, N, K, A, 1 << 19, B, N, C, N))
    assert small["mode"] == sg.SGEMM_MODE_EDGE
    lda = (1 << 25) + (1 << 22) + 3  # 31 rows of it (32-row tiles) exceed 4 GiB
    huge = sg.sgemm_kernel_info(sg.sgemm_select_kernel(0, M, N, K, A, lda, B, N, C, N))
    assert huge["mode"] == sg.SGEMM_MODE_GUARDED
    # the same through B's stride (B stored as K x N: K-step rows of ldb)
    ldb = (1 << 28) + 3
    huge_b = sg.sgemm_kernel_info(sg.sgemm_select_kernel(0, M, N, K, A, K, B, ldb, C, N))
    assert huge_b["mode"] == sg.SGEMM_MODE_GUARDED


def test_stream_k_instances_and_schedules():
    """Every MFMA tile shape but 256x256 (whose stream-K kernel would not fit
    its registers) and 32x64 (three resident one-tile workgroups per CU
    already balance the CUs) has stream-K instances for every storage in the
    aligned and edge modes; the host-only planners never pick them (they
    plan without a workspace)."""
    table = sg.kernel_table()
    assert sg.library().sgemm_kernel_schedule(-1) == sg.SGEMM_ERR_VALUE
    sk = [k for k in table if k["schedule"] == sg.SGEMM_SCHEDULE_STREAM_K]
    assert sk and all(k["variant"] == sg.SGEMM_VARIANT_MFMA for k in sk)
    assert all(k["mode"] in (sg.SGEMM_MODE_ALIGNED, sg.SGEMM_MODE_EDGE) for k in sk)
    shapes = {(k["bm"], k["bn"], k["bk"]) for k in table if k["variant"] == sg.SGEMM_VARIANT_MFMA}
    assert not any((k["bm"], k["bn"]) in ((256, 256), (32, 64)) for k in sk)
    for shape in (s for s in shapes if s[:2] not in ((256, 256), (32, 64))):
        got = {(k["transa"], k["transb"], k["mode"]) for k in sk
               if (k["bm"], k["bn"], k["bk"]) == shape}
        assert got == {(a, b, m) for a in (0, 1) for b in (0, 1)
                       for m in (sg.SGEMM_MODE_ALIGNED, sg.SGEMM_MODE_EDGE)}, shape
    A, B, C = 0x10000000, 0x20000000, 0x40000000
    for M, N, K in ((4100, 4100, 4100), (1000, 1500, 777)):
        for kid, _, _ in sg.sgemm_plan(0, M, N, K, A, K, B, N, C, N):
            assert sg.sgemm_kernel_schedule(kid) == sg.SGEMM_SCHEDULE_TILES


def test_workspace_calls_without_a_device():
    """Null-handle and argument errors of the workspace calls (no GPU)."""
    lib = sg.library()
    import ctypes
    n = ctypes.c_size_t()
    assert lib.sgemm_workspace_size(None, ctypes.byref(n)) == sg.SGEMM_ERR_HANDLE
    assert lib.sgemm_set_workspace(None, None, 0) == sg.SGEMM_ERR_HANDLE
    assert lib.sgemm_plan_handle(None, 0, 0, 8, 8, 8, None, 8, None, 8, None, 8,
                                 None, None) == sg.SGEMM_ERR_HANDLE


def test_plans_follow_measured_winners():
    """Shapes where the launch-time model must pick what measured fastest on
    MI355X: 4096 x 11008 x 4096 as five rounds of 256x128 then 64x64 tiles
    (2461 us, against 2620 for one 128x128 launch), 8192^2 x 4096 on 256x128
    (96% of peak), 1024^3 on 32x64 (19.8 against 20.5 us on 64x64), 3000^3
    on 64x64."""
    A, B, C = 0x10000000, 0x20000000, 0x40000000
    name = lambda M, N, K: [sg.sgemm_kernel_name(k) for k, _, _ in
                            sg.sgemm_plan(0, M, N, K, A, K, B, N, C, N)]
    assert name(4096, 11008, 4096) == ["mfma_M256x128_aligned", "mfma_M64x64_aligned"]
    assert name(8192, 8192, 4096) == ["mfma_M256x128_aligned"]
    assert name(1024, 1024, 1024) == ["mfma_M32x64_aligned"]
    assert name(1000, 1500, 777) == ["mfma_M32x64_edge"]
    assert name(3000, 3000, 3000) == ["mfma_M64x64_edge"]


@pytest.mark.parametrize("tb", [0, 1])
def test_decode_shapes_plan_the_one_pass_kernels(tb):
    """Without a workspace (the host-only planner), decode-like products with
    up to 8 rows of A take the one-pass kernel with the fewest rows that hold
    M, for B stored N x K (valu_S<MT>_nt_small) and as stored
    (valu_S<MT>x32_small); 9 rows do not."""
    A, B, C = 0x10000000, 0x20000000, 0x40000000
    for M, N, K in ((1, 4096, 4096), (2, 4096, 4096), (3, 11008, 4096), (8, 4096, 4096),
                    (5, 14336, 4096), (1, 4096, 14336)):
        mt = next(m for m in (1, 2, 4, 8) if m >= M)
        kid = sg.sgemm_select_kernel(0, M, N, K, A, K, B, K if tb else N, C, N) if not tb \
            else sg.sgemm_plan(0, M, N, K, A, K, B, K, C, N, transb=1)[0][0]
        want = f"valu_S{mt}_nt_small" if tb else f"valu_S{mt}x32_small"
        assert sg.sgemm_kernel_name(kid) == want, (M, N, K, tb, sg.sgemm_kernel_name(kid))
    plan = sg.sgemm_plan(0, 9, 4096, 4096, A, 4096, B, 4096, C, 4096, transb=tb)
    name = sg.sgemm_kernel_name(plan[0][0])
    assert not (name.startswith("valu_S") and name.endswith("_nt_small")) and "x32_" not in name


def test_small_m_plans():
    """A few rows of A against a wide B plan the small-M kernel with the
    fewest rows that hold M, for every storage (up to 16 rows with B as
    stored, one pass up to 8; 8 with B transposed); more rows or an explicit
    MFMA variant never do."""
    A, B, C = 0x10000000, 0x20000000, 0x40000000
    def plan(M, N, K, variant=0, ta=0, tb=0):
        lda = M if ta else K
        ldb = K if tb else N
        return [sg.sgemm_kernel_info(k) for k, _, _ in
                sg.sgemm_plan(variant, M, N, K, A, lda, B, ldb, C, N, transa=ta, transb=tb)]
    for M, bm, bm_t in ((1, 1, 1), (2, 2, 2), (4, 4, 4), (5, 8, 8), (16, 16, None)):
        for ta in (0, 1):
            for tb in (0, 1):
                if tb and bm_t is None:
                    continue
                # no workspace here: one K range for B as stored, so a wide B
                p = plan(M, 4096, 16384, ta=ta, tb=tb) if tb else plan(M, 65536, 1024, ta=ta)
                assert [(k["schedule"], k["bm"], k["transa"], k["transb"]) for k in p] == \
                    [(sg.SGEMM_SCHEDULE_SMALL_M, bm_t if tb else bm, ta, tb)], (M, ta, tb)
    assert plan(17, 65536, 1024)[0]["schedule"] != sg.SGEMM_SCHEDULE_SMALL_M
    assert plan(9, 4096, 16384, tb=1)[0]["schedule"] != sg.SGEMM_SCHEDULE_SMALL_M
    assert plan(4, 65536, 1024, variant=sg.SGEMM_VARIANT_MFMA)[0]["variant"] == \
        sg.SGEMM_VARIANT_MFMA
    assert plan(4, 65536, 1024, variant=sg.SGEMM_VARIANT_VALU)[0]["schedule"] == \
        sg.SGEMM_SCHEDULE_SMALL_M
