"""Seeded input generators: determinism, ranges, layout."""
import numpy as np

from fp32_gemm_major_amd import workloads as wl


def test_deterministic_and_seeded_by_role():
    a1 = wl.draw(3, wl.ROLE_A, 64, 48, "uniform")
    a2 = wl.draw(3, wl.ROLE_A, 64, 48, "uniform")
    b = wl.draw(3, wl.ROLE_B, 64, 48, "uniform")
    assert a1.dtype == np.float32 and a1.tobytes() == a2.tobytes()
    assert not np.array_equal(a1, b)


def test_uniform_grid_and_range():
    a = wl.draw(1, wl.ROLE_A, 256, 256, "uniform")
    assert a.min() >= -1.0 and a.max() < 1.0
    # values lie on the 2^-23 grid, so they are exact FP32 numbers
    scaled = a.astype(np.float64) * 2.0 ** 23
    assert np.array_equal(scaled, np.round(scaled))


def test_int4_and_normal():
    i = wl.draw(101, wl.ROLE_A, 128, 128, "int4")
    assert set(np.unique(i)) <= set(range(-4, 5)) and len(np.unique(i)) == 9
    n = wl.draw(5, wl.ROLE_B, 512, 512, "normal")
    assert abs(float(n.std()) - 0.02) < 0.001 and abs(float(n.mean())) < 0.001


def test_leading_dims_keep_values_and_pad():
    w = wl.WORKLOADS["c4_edge"]
    o1 = wl.operands(w, M=10, N=12, K=7)
    o2 = wl.operands(w, M=10, N=12, K=7, lda=9, ldb=16, ldc=13)
    assert np.array_equal(o1.A.reshape(10, 7), o2.A.reshape(10, 9)[:, :7])
    assert np.all(np.isnan(o2.A.reshape(10, 9)[:, 7:]))
    assert np.array_equal(o1.C.reshape(10, 12), o2.C.reshape(10, 13)[:, :12])


def test_registry_matches_configs():
    w = wl.WORKLOADS
    assert (w["c3_4096"].M, w["c3_4096"].N, w["c3_4096"].K) == (4096, 4096, 4096)
    assert (w["c3_4096"].alpha, w["c3_4096"].beta) == (1.5, 0.5)
    assert (w["c4_edge"].M, w["c4_edge"].N, w["c4_edge"].K) == (1000, 1500, 777)
    assert (w["c5_mlp"].N, w["c5_mlp"].dist) == (11008, "normal")
    assert w["c2_1024"].c_fill == "nan" and w["c2_1024"].beta == 0.0
