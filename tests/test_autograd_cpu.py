"""The autograd wrapper's host-side behaviour (no GPU needed)."""
import pytest
import torch

from linear_cross_entropy_cce_amd import LinearCrossEntropy, linear_cross_entropy


def test_rejects_unknown_reduction():
    E = torch.zeros(4, 8)
    with pytest.raises(ValueError):
        linear_cross_entropy(E, torch.zeros(5, 8), torch.zeros(4, dtype=torch.int64),
                             reduction="avg")
    with pytest.raises(ValueError):
        LinearCrossEntropy(reduction="avg")


def test_rejects_host_tensors_before_any_library_call():
    E = torch.zeros(4, 8)
    with pytest.raises(ValueError, match="GPU tensor"):
        linear_cross_entropy(E, torch.zeros(5, 8), torch.zeros(4, dtype=torch.int64),
                             reduction="none")
