"""matmul(): the operand layout chosen from strides (pure host logic, CPU)."""
import pytest
import torch

import dense_fp16_gemm_amd as g


@pytest.mark.parametrize("ta,tb,want", [(False, False, "nn"), (False, True, "nt"),
                                        (True, False, "tn"), (True, True, "tt")])
def test_layout_from_strides(ta, tb, want):
    m, n, k = 5, 7, 3
    a = torch.zeros(k, m).t() if ta else torch.zeros(m, k)
    b = torch.zeros(n, k).t() if tb else torch.zeros(k, n)
    lay, xa, xb = g.matmul_layout(a, b)
    assert lay == want
    assert xa.is_contiguous() and xb.is_contiguous()
    # the stored matrices are the ones gemm() takes for that layout
    assert tuple(xa.shape) == ((k, m) if ta else (m, k))
    assert tuple(xb.shape) == ((n, k) if tb else (k, n))
    assert xa.data_ptr() == a.data_ptr() and xb.data_ptr() == b.data_ptr(), "no copies"


def test_other_strides_rejected():
    a = torch.zeros(6, 8)[:, ::2]           # a column stride of 2
    with pytest.raises(ValueError, match="row-major"):
        g.matmul_layout(a, torch.zeros(4, 3))
    with pytest.raises(ValueError, match="matrices"):
        g.matmul_layout(torch.zeros(2, 3, 4), torch.zeros(4, 3))


def test_matmul_checks_inner_dimensions():
    with pytest.raises(ValueError, match="shape mismatch"):
        g.matmul(torch.zeros(4, 3, dtype=torch.float16), torch.zeros(5, 2, dtype=torch.float16))
