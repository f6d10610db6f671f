"""Seeded input generators: determinism, ranges, layout."""
import numpy as np
import pytest

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


def test_round16_nearest_even():
    """The 16-bit input rounding agrees with library conversions (torch's
    bfloat16, numpy's float16), ties included."""
    import torch
    rng = np.random.default_rng(5)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    ties = np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130,
                       1 + 2 ** -11, 1 + 3 * 2 ** -11, 0.0, -0.0, 65504.0, 3e38])
    x = np.concatenate([x, ties])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(wl.round16(x, "bf16"), want.view(np.uint16))
    assert np.array_equal(wl.round16(x[:-1], "f16"),
                          x[:-1].astype(np.float16).view(np.uint16))
    with pytest.raises(ValueError):
        wl.round16(np.float32([np.nan]), "bf16")


def test_operands16_values():
    """16-bit operands hold the rounded FP32 draws; storage flags transpose."""
    w = wl.WORKLOADS["c4_edge"]
    o = wl.operands16(w, "bf16", M=40, N=24, K=33)
    o_t = wl.operands16(w, "bf16", M=40, N=24, K=33, ta=True, tb=True)
    a = o.A.reshape(40, 33)
    assert np.array_equal(a, wl.round16(wl.draw(w.cfg_id, wl.ROLE_A, 40, 33, w.dist), "bf16"))
    assert np.array_equal(o_t.A.reshape(33, 40).T, a)
    assert np.array_equal(o_t.B.reshape(24, 33).T, o.B.reshape(33, 24))
    assert o.C.dtype == np.float32 and o.A.dtype == np.uint16


def test_round8_nearest_even():
    """The 8-bit input rounding is torch's (checked here against an exact
    nearest-even search over each format's finite values)."""
    import torch
    from fractions import Fraction
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(3000) * 3.0).astype(np.float32)
    for dt, tdt in (("fp8e4m3", torch.float8_e4m3fn), ("fp8e5m2", torch.float8_e5m2)):
        bits = wl.round8(x, dt)
        allv = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(tdt).double().numpy()
        finite = [(abs(float(v)), b) for b, v in enumerate(allv) if np.isfinite(v) and b < 128]
        for xi, bi in zip(x[:400], bits[:400]):
            a = abs(float(xi))
            best = min(finite, key=lambda vb: (abs(Fraction(vb[0]) - Fraction(a)), vb[1] & 1))
            got = float(allv[bi])
            assert abs(got) == best[0] and (got == 0 or np.sign(got) == np.sign(xi)), (dt, xi)
    with pytest.raises(ValueError):
        wl.round8(np.float32([1000.0]), "fp8e4m3")
