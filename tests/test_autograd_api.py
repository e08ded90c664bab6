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


def test_layout_views_are_passed_without_copies():
    import torch

    from io_aware_exact_24_amd import autograd, binding

    x = torch.zeros(2, 100, 4, 64, dtype=torch.bfloat16)  # [B, N, H, d]
    v = autograd._to_bhnd(x, "bnhd")
    assert v.shape == (2, 4, 100, 64) and v.data_ptr() == x.data_ptr()
    assert v.stride() == (100 * 4 * 64, 64, 4 * 64, 1)
    c = torch.zeros(2, 4, 100, 64, dtype=torch.float16)
    assert autograd._to_bhnd(c, "bhnd").data_ptr() == c.data_ptr()
    # a fused QKV projection [B, N, 3, H, d]: each of q, k, v is read in place
    qkv = torch.zeros(2, 100, 3, 4, 64, dtype=torch.bfloat16)
    q = autograd._to_bhnd(qkv[:, :, 0], "bnhd")
    assert q.data_ptr() == qkv.data_ptr() and q.stride(2) == 3 * 4 * 64
    # what the strided entry points cannot address is copied
    e = torch.zeros(1, 1, 1, 64, dtype=torch.bfloat16).expand(2, 4, 100, 64)
    assert not binding.kernel_layout_ok(e)
    assert autograd._to_bhnd(e, "bhnd").is_contiguous()
    odd = torch.zeros(2, 4, 100, 72, dtype=torch.bfloat16)[..., 4:68]  # rows start 8 bytes in
    assert not binding.kernel_layout_ok(odd)
