"""CPU: argument handling of the autograd entry point that needs no GPU."""

import pytest
import torch

from io_aware_exact_24_amd.autograd import flash_attention, scaled_dot_product_attention


def test_attn_mask_is_rejected_before_any_launch():
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(NotImplementedError):
        scaled_dot_product_attention(q, q, q, attn_mask=torch.ones(4, 4, dtype=torch.bool))


def test_unknown_layout_is_rejected():
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        flash_attention(q, q, q, layout="nhd")
