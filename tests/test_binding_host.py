"""Host-side checks of the Python binding that run before any library call
(no GPU): a grad_output of the wrong length is refused, since the kernels
read exactly one value, or one per row, from it."""
import pytest
import torch

from softmax_cross_entropy_amd import backward_, backward_recompute


def _recompute(go, reduction, rows=5, V=16):
    x = torch.zeros((rows, V))
    t = torch.zeros(rows, dtype=torch.int64)
    stats = torch.zeros((rows, 2))
    return backward_recompute(x, t, None, -100, 0.0, 0.0, None, reduction, stats, go)


@pytest.mark.parametrize("go", [torch.tensor(1.0), torch.ones(4), torch.ones(6)])
def test_recompute_none_needs_one_grad_output_per_row(go):
    with pytest.raises(ValueError, match="one per row"):
        _recompute(go, "none")


@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_recompute_reduced_needs_a_scalar_grad_output(reduction):
    with pytest.raises(ValueError, match="a scalar"):
        _recompute(torch.ones(5), reduction)


def test_backward_per_row_length_checked():
    g = torch.zeros((5, 16))
    with pytest.raises(ValueError, match="one per row"):
        backward_(g, torch.tensor(2.0), per_row=True)
    with pytest.raises(ValueError, match="a scalar"):
        backward_(g, torch.ones(5), per_row=False)
