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


def test_split_count_per_shape():
    from io_aware_exact_24_amd.autograd import split_count

    cus = 256
    # shapes that fill the GPU with the plain forward take no split
    assert split_count(4, 32, 4096, 128, True, cus) == 0
    assert split_count(8, 16, 1024, 64, False, cus) == 0
    # few query blocks: shares for one workgroup per CU (causal: two), at least 2 ...
    assert split_count(1, 1, 4096, 128, True, cus) == 8    # 64 tiles: 8 shares of 8
    assert split_count(1, 8, 2048, 64, False, cus) == 2    # 128 blocks x 2 = 256
    assert split_count(1, 4, 8192, 128, True, cus) == 2    # 256 blocks x 2 = 512 = 2 per CU
    assert split_count(1, 2, 8192, 64, True, cus) == 4     # 128 blocks x 4 = 512
    # ... but at least eight 64-key tiles per share, and at most FA_MAX_SPLITS
    assert split_count(1, 2, 1000, 128, True, cus) == 2    # 16 tiles -> 2 shares of 8
    assert split_count(2, 4, 1024, 128, False, cus) == 0   # 16 tiles, 64 workgroups
    assert split_count(1, 3, 4096, 64, False, cus) == 2    # 96 blocks: 2 shares fill the CUs
    assert split_count(1, 1, 128, 64, False, cus) == 0     # 2 tiles: nothing to split
    assert split_count(1, 1, 1 << 16, 128, False, 1 << 15) == 64
    # only the MFMA head sizes have a split forward
    assert split_count(1, 1, 4096, 96, True, cus) == 0


def test_backward_split_count_per_shape():
    from io_aware_exact_24_amd.autograd import backward_split_count

    cus = 256
    # enough units already: the plain backward
    assert backward_split_count(4, 32, 4096, 128, True, cus) == 0
    assert backward_split_count(8, 16, 1024, 64, False, cus) == 0
    # too few units: shares until the units cover the CUs, four tiles each at least
    assert backward_split_count(1, 8, 4096, 128, True, cus) == 2    # 128 causal pairs
    assert backward_split_count(1, 1, 4096, 128, True, cus) == 16   # 16 pairs of 66 tiles
    assert backward_split_count(1, 4, 2048, 64, False, cus) == 4    # 64 blocks of 32 tiles
    assert backward_split_count(1, 2, 1000, 128, True, cus) == 4    # 8 pairs of 18 tiles
    assert backward_split_count(1, 2, 300, 64, True, cus) == 0      # 7 tiles: nothing to split
    assert backward_split_count(1, 1, 4096, 96, True, cus) == 0     # generic kernels: no split
    # half the CUs busy: two shares only for long units
    assert backward_split_count(2, 8, 2048, 128, True, cus) == 0    # 128 pairs of 34 tiles
    assert backward_split_count(1, 16, 1024, 64, False, cus) == 0   # 128 blocks of 16 tiles
