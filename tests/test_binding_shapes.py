"""The torch-tensor binding refuses calls whose tensors cannot hold the
windows the kernels would touch (CPU tensors: the check is pure host logic
and runs before anything reaches a device)."""
import pytest

torch = pytest.importorskip("torch")

from fp32_gemm_major_amd import _shapes, check_extents  # noqa: E402


def t(*shape):
    return torch.zeros(*shape, dtype=torch.float32)


def test_sizes_from_2d_tensors():
    assert _shapes(t(5, 7), t(7, 3), t(5, 3), None, None, None, None, None, None,
                   False, False) == (5, 3, 7, 7, 3, 3)
    # transposed storage: A stored K x M, B stored N x K
    assert _shapes(t(7, 5), t(3, 7), t(5, 3), None, None, None, None, None, None,
                   True, True) == (5, 3, 7, 5, 7, 3)


def test_b_rows_disagree_with_a():
    with pytest.raises(ValueError, match="disagree on K"):
        _shapes(t(5, 7), t(6, 3), t(5, 3), None, None, None, None, None, None, False, False)
    # an explicit K that both hold is fine; one that B cannot hold is not
    assert _shapes(t(5, 7), t(8, 3), t(5, 3), None, None, 7, None, None, None,
                   False, False)[2] == 7
    with pytest.raises(ValueError, match="B"):
        _shapes(t(5, 9), t(8, 3), t(5, 3), None, None, 9, None, None, None, False, False)


def test_short_c():
    with pytest.raises(ValueError, match="C"):
        _shapes(t(5, 7), t(7, 3), t(4, 3), None, None, None, None, None, None, False, False)
    with pytest.raises(ValueError, match="C"):
        _shapes(t(5, 7), t(7, 3), t(5, 2), None, None, None, None, None, None, False, False)
    # a 1-D C shorter than (M-1)*ldc + N
    with pytest.raises(ValueError, match="C"):
        _shapes(t(5, 7), t(7, 3), t(14), None, None, None, None, None, 3, False, False)
    assert _shapes(t(5, 7), t(7, 3), t(15), None, None, None, None, None, 3,
                   False, False)[5] == 3


def test_explicit_sizes_larger_than_tensors():
    with pytest.raises(ValueError, match="A"):
        _shapes(t(5, 7), t(7, 3), t(9, 3), 9, None, None, None, None, None, False, False)
    with pytest.raises(ValueError, match="B"):
        _shapes(t(5, 7), t(7, 3), t(5, 4), None, 4, None, None, None, None, False, False)


def test_1d_buffers_and_views_count_storage_from_the_pointer():
    buf = t(100)
    # a view that starts 10 elements in: 90 elements remain
    check_extents(buf[10:], t(80), t(72), 9, 8, 10, 10, 8, 8, False, False)
    with pytest.raises(ValueError, match="A"):
        check_extents(buf[11:], t(80), t(72), 9, 8, 10, 10, 8, 8, False, False)
    # a 2-D view whose rows are strided inside a larger buffer
    big = t(8, 12)
    C = big[:, :5]
    assert _shapes(t(8, 3), t(3, 5), C, None, None, None, None, None, None,
                   False, False)[5] == 12


def test_untouched_operands_are_not_checked():
    # K = 0: A and B are not read; M = 0: nothing is touched
    check_extents(t(1), t(1), t(20), 4, 5, 0, 1, 5, 5, False, False)
    check_extents(t(1), t(1), t(1), 0, 5, 7, 7, 5, 5, False, False)
    with pytest.raises(ValueError, match="C"):
        check_extents(t(1), t(1), t(19), 4, 5, 0, 1, 5, 5, False, False)


def test_16_and_8_bit_element_sizes():
    A = torch.zeros(5, 7, dtype=torch.bfloat16)
    B = torch.zeros(3, 7, dtype=torch.float8_e4m3fn)
    assert _shapes(A, torch.zeros(7, 3, dtype=torch.bfloat16), t(5, 3), None, None, None,
                   None, None, None, False, False) == (5, 3, 7, 7, 3, 3)
    with pytest.raises(ValueError, match="B"):
        check_extents(torch.zeros(35, dtype=torch.float8_e4m3fn), B.reshape(-1)[1:], t(15),
                      5, 3, 7, 7, 7, 3, False, True)
