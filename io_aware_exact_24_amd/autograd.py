"""PyTorch autograd entry point over the C ABI (argument marshalling only).

`flash_attention` runs fa_fwd (fa_fwd_split when the shape has too few query
blocks to fill the GPU) in the forward of a torch.autograd.Function and fa_bwd
(fa_bwd_split when it has too few key blocks) in its backward, keeping only
what the recompute backward needs: Q, K, V, O and the per-row log-sum-exp (no
N x N matrix; ML Canon 48 FlashAttention, "backward without N x N").  `scaled_dot_product_attention` takes the argument
names of torch.nn.functional.scaled_dot_product_attention, the drop-in call the
same page shows, for the cases the library computes.

The kernels take [B, H, N, d] tensors of any batch, head and row strides
(last dimension contiguous, rows 16-byte aligned).  layout="bnhd" accepts
[B, N, H, d] (the layout of a fused QKV projection) and returns O in it: the
tensors go to the library as transposed views, O, dQ, dK and dV are
allocated in the inputs' memory layout, and nothing is copied.  A tensor the
strided entry points cannot address in place (e.g. an expanded gradient with
zero strides) is copied to contiguous memory first.
"""

import torch

from . import binding


def _in_place(t):
    """t itself when the library can address it, else a contiguous copy."""
    return t if binding.kernel_layout_ok(t) else t.contiguous()


def _to_bhnd(t, layout):
    if layout == "bhnd":
        return _in_place(t)
    if layout == "bnhd":
        return _in_place(t.transpose(1, 2))
    raise ValueError(f"layout must be 'bhnd' or 'bnhd', not {layout!r}")


def _from_bhnd(t, layout):
    return t if layout == "bhnd" else t.transpose(1, 2)


def split_count(B, H, N, d, causal, cus):
    """Key splits for the forward of one shape (0: the plain fa_fwd).

    The plain forward launches one workgroup per 128-query block (causal ones
    in pairs, so each has the same work), two per CU.  When that leaves CUs
    idle, the split forward (one workgroup per query block and key share)
    takes as many shares as fit one workgroup per CU, two with a causal mask
    (its blocks have unequal work, which more shares even out), at least 2;
    each share keeps at least eight 64-key tiles of the longest block, and
    there are at most FA_MAX_SPLITS.  Short sequences (under 32 key tiles)
    are split only when the plain grid is tiny (16 workgroups or fewer):
    otherwise the combine pass costs more than the shorter shares save.
    Only the MFMA head sizes have a split forward.  (Rules fitted to
    back-to-back timings of both passes over 16 shapes.)
    """
    if d not in (64, 128):
        return 0
    blocks = (N + 127) // 128
    plain = B * H * ((blocks + 1) // 2 if causal else blocks)
    if plain >= cus:
        return 0
    tiles = (N + 63) // 64
    if tiles < 32 and plain > 16:
        return 0
    want = max(2, (2 if causal else 1) * cus // (B * H * blocks))
    cap = min(max(tiles // 8, 1), binding.FA_MAX_SPLITS)
    s = min(want, cap)
    return s if s >= 2 else 0


def backward_split_count(B, H, N, d, causal, cus):
    """Shares for the backward of one shape (0: the plain fa_bwd).

    The dK/dV stage runs one persistent workgroup per CU over work units of
    one 128-key block (with a causal mask, a pair of blocks of equal total
    work).  When there are fewer units than CUs, fa_bwd_split cuts each
    unit's query tiles (and each query block's key tiles for dQ) into as many
    shares as keep one unit per CU, at least 2, each with at least four
    64-row tiles, at most FA_MAX_SPLITS.  With half the CUs or more already
    busy, two shares pay only for long units (64 tiles or more).  Only the
    MFMA head sizes have a split backward.  (Rules fitted to back-to-back
    timings of both passes over 16 shapes.)
    """
    if d not in (64, 128):
        return 0
    blocks = (N + 127) // 128
    units = B * H * ((blocks + 1) // 2 if causal else blocks)
    if units >= cus:
        return 0
    tiles = (N + 63) // 64
    per_unit = tiles + 2 if causal else tiles  # a causal pair's tiles, both blocks
    if 2 * units >= cus and per_unit < 64:
        return 0
    want = max(2, cus // units)
    cap = min(max(per_unit // 4, 1), binding.FA_MAX_SPLITS)
    s = min(want, cap)
    return s if s >= 2 else 0


def _splits(q, causal):
    """split_count for q's shape on its GPU: 16-bit types, contiguous tensors
    only (the split entry point takes no strides)."""
    if q.dtype not in (torch.bfloat16, torch.float16) or not q.is_cuda or not q.is_contiguous():
        return 0
    B, H, N, d = q.shape
    cus = torch.cuda.get_device_properties(q.device).multi_processor_count
    return split_count(B, H, N, d, causal, cus)


def _forward(q, k, v, scale, causal, key_lens, dropout_p, seed):
    s = _splits(q, causal) if k.is_contiguous() and v.is_contiguous() else 0
    if s:
        return binding.forward_split(q, k, v, scale, causal, key_lens, dropout_p, seed, s)
    return binding.forward(q, k, v, scale, causal, key_lens, dropout_p, seed)


def _bwd_splits(q, causal, tensors):
    """backward_split_count for q's shape on its GPU: 16-bit types, every
    tensor contiguous (the split entry point takes no strides)."""
    if q.dtype not in (torch.bfloat16, torch.float16) or not q.is_cuda:
        return 0
    if not all(t.is_contiguous() for t in tensors):
        return 0
    B, H, N, d = q.shape
    cus = torch.cuda.get_device_properties(q.device).multi_processor_count
    return backward_split_count(B, H, N, d, causal, cus)


class FlashAttentionFunction(torch.autograd.Function):
    """O = softmax(mask(scale * Q K^T)) (with dropout) V on [B, H, N, d]."""

    @staticmethod
    def forward(ctx, q, k, v, scale, causal, key_lens, dropout_p, seed):
        o, lse = _forward(q, k, v, scale, causal, key_lens, dropout_p, seed)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.key_lens = key_lens
        ctx.args = (scale, causal, dropout_p, seed)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        scale, causal, dropout_p, seed = ctx.args
        do = _in_place(do)
        s = _bwd_splits(q, causal, (q, k, v, o, do))
        if s:
            dq, dk, dv = binding.backward_split(q, k, v, o, do, lse, scale, causal, ctx.key_lens,
                                                dropout_p, seed, s)
        else:
            dq, dk, dv = binding.backward(q, k, v, o, do, lse, scale, causal, ctx.key_lens,
                                          dropout_p, seed)
        return dq, dk, dv, None, None, None, None, None


def flash_attention(q, k, v, scale=None, causal=False, key_lens=None, dropout_p=0.0, seed=None,
                    layout="bhnd"):
    """Exact attention with autograd support.

    q, k, v: bf16, fp16 or fp32 CUDA tensors [B, H, N, d] (layout="bhnd") or
    [B, N, H, d] (layout="bnhd"), d in {32, 64, 96, 128, 256}, read in place
    (16-bit d = 64 and 128 run on the MFMA kernels, the rest on the generic
    ones; fp32 takes no dropout).  scale defaults to 1/sqrt(d).  key_lens: int32 [B]
    (device or host) masking keys j >= key_lens[b].  dropout_p > 0 draws a
    Philox seed from torch's default CPU generator when seed is None; the same
    seed is replayed in the backward.
    """
    d = q.shape[-1]
    if scale is None:
        scale = d ** -0.5
    if seed is None:
        seed = int(torch.randint(0, 2**62, (1,)).item()) if dropout_p > 0.0 else 0
    if key_lens is not None:
        key_lens = key_lens.to(device=q.device, dtype=torch.int32)
    qb, kb, vb = (_to_bhnd(t, layout) for t in (q, k, v))
    if torch.is_grad_enabled() and any(t.requires_grad for t in (q, k, v)):
        o = FlashAttentionFunction.apply(qb, kb, vb, float(scale), bool(causal), key_lens,
                                         float(dropout_p), int(seed))
    else:
        o, _ = _forward(qb, kb, vb, float(scale), bool(causal), key_lens, float(dropout_p),
                        int(seed))
    return _from_bhnd(o, layout)


def scaled_dot_product_attention(query, key, value, attn_mask=None, dropout_p=0.0,
                                 is_causal=False, scale=None):
    """torch.nn.functional.scaled_dot_product_attention's arguments on [B, H, N, d].

    attn_mask is not supported (use flash_attention's key_lens for key
    padding); a causal mask is square and top-left, key j visible to query i
    iff j <= i.
    """
    if attn_mask is not None:
        raise NotImplementedError("attn_mask is not supported; use flash_attention(key_lens=...)")
    return flash_attention(query, key, value, scale=scale, causal=is_causal, dropout_p=dropout_p)
