"""GPU tests of the strided entry points (fa_fwd_strided, fa_bwd_strided) and of
fp16.

The strided kernels run the same arithmetic as the contiguous ones, so on
the same values their outputs must be equal bit for bit; the only thing that
changes is where rows are read and written.  Outputs are allocated with
sentinel-filled gaps between rows and heads, which must come back untouched.
fp16 is checked against the fp64 oracle under the bf16 tolerances.
"""

import math

import numpy as np
import pytest
import torch

from fa_testlib import DEV, TOL_GRAD, TOL_LSE, TOL_O, f64, max_abs, note, rel_l2
from io_aware_exact_24_amd import autograd, binding
from io_aware_exact_24_amd.workloads import draw
from oracle import attention_backward, attention_forward

pytestmark = pytest.mark.gpu

SENTINEL = -12345.0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def alloc(shape, dtype, kind):
    """An uninitialised-looking [B, H, N, d] view in memory of the given kind,
    with every element outside the view set to SENTINEL; returns (view, buffer)."""
    B, H, N, d = shape
    if kind == "bhnd":
        buf = torch.full((B, H, N, d), SENTINEL, dtype=dtype, device=DEV)
        return buf, buf
    if kind == "bnhd":
        buf = torch.full((B, N, H, d), SENTINEL, dtype=dtype, device=DEV)
        return buf.transpose(1, 2), buf
    if kind == "gaps":  # rows 24 elements apart beyond d, heads 2 rows apart beyond N
        buf = torch.full((B, H, N + 2, d + 24), SENTINEL, dtype=dtype, device=DEV)
        return buf[:, :, 1:N + 1, 8:d + 8], buf
    raise ValueError(kind)


def place(t, kind):
    """t's values in memory of the given kind (a [B, H, N, d] view)."""
    view, _ = alloc(t.shape, t.dtype, kind)
    view.copy_(t.to(DEV))
    return view


def qkv_views(q, k, v):
    """q, k, v as views of one fused [B, N, 3, H, d] projection buffer."""
    B, H, N, d = q.shape
    buf = torch.empty((B, N, 3, H, d), dtype=q.dtype, device=DEV)
    for i, t in enumerate((q, k, v)):
        buf[:, :, i].copy_(t.to(DEV).transpose(1, 2))
    return tuple(buf[:, :, i].transpose(1, 2) for i in range(3)), buf


def untouched(buf, view):
    """Every element of buf outside view still holds SENTINEL."""
    mask = torch.ones(buf.shape, dtype=torch.bool, device=DEV)
    inner = torch.as_strided(mask, view.shape, view.stride(),
                             view.storage_offset() - buf.storage_offset())
    inner.fill_(False)
    return bool((buf[mask] == SENTINEL).all())


CASES = [
    # dtype, d, causal, padded, p
    (torch.bfloat16, 128, True, False, 0.0),
    (torch.bfloat16, 128, False, True, 0.1),
    (torch.bfloat16, 64, False, False, 0.0),
    (torch.bfloat16, 64, True, True, 0.2),
    (torch.float16, 128, True, True, 0.0),
    (torch.float16, 64, False, False, 0.1),
]


def case_id(c):
    dt, d, causal, padded, p = c
    return "{}-d{}{}{}{}".format("bf16" if dt == torch.bfloat16 else "fp16", d,
                                 "-causal" if causal else "", "-pad" if padded else "",
                                 f"-p{p}" if p else "")


@pytest.mark.parametrize("kind", ["bnhd", "gaps", "qkv"])
@pytest.mark.parametrize("case", CASES, ids=case_id)
def test_strided_equals_contiguous(case, kind):
    dt, d, causal, padded, p = case
    B, H, N, seed = 2, 3, 300, 0xC0FFEE
    note(f"strided {kind} {case_id(case)} B{B} H{H} N{N}")
    inp = draw(B, H, N, d, dt, seed=CASES.index(case) + 7, padded=padded)
    scale = float(np.float32(1 / math.sqrt(d)))
    q, k, v, do = (t.to(DEV) for t in (inp.q, inp.k, inp.v, inp.dout))
    kl = None if inp.key_lens is None else inp.key_lens.to(DEV)
    # the contiguous path
    o_c, lse_c = binding.forward(q, k, v, scale, causal, kl, p, seed)
    g_c = binding.backward(q, k, v, o_c, do, lse_c, scale, causal, kl, p, seed)
    # the same values laid out by strides
    if kind == "qkv":
        (qs, ks, vs), _ = qkv_views(q, k, v)
        okind = "bnhd"
    else:
        qs, ks, vs = (place(t, kind) for t in (q, k, v))
        okind = kind
    o_s, o_buf = alloc(q.shape, dt, okind)
    lse_s = torch.empty_like(lse_c)
    binding.fa_fwd_strided(qs, ks, vs, o_s, lse_s, scale, causal, kl, p, seed)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_c) and torch.equal(lse_s, lse_c)
    assert untouched(o_buf, o_s)
    dos = place(do, okind)
    if kind == "qkv":  # gradients into one fused [B, N, 3, H, d] buffer, as a QKV backward would
        gbuf = torch.full((B, N, 3, H, d), SENTINEL, dtype=dt, device=DEV)
        gs = [gbuf[:, :, i].transpose(1, 2) for i in range(3)]
        bufs = [gbuf] * 3
    else:
        pairs = [alloc(q.shape, dt, kind) for _ in range(3)]
        gs, bufs = [pp[0] for pp in pairs], [pp[1] for pp in pairs]
    nbytes = binding.fa_bwd_workspace_size(B, H, N, d, binding._dtype_code(q))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    binding.fa_bwd_strided(qs, ks, vs, o_s, dos, lse_s, gs[0], gs[1], gs[2], scale, causal, kl, p,
                           seed, ws)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), gs, g_c):
        assert torch.equal(a, b), name
    if kind == "qkv":
        assert bool((gbuf != SENTINEL).all())  # the three views tile the buffer
    else:
        for name, buf, view in zip(("dq", "dk", "dv"), bufs, gs):
            assert untouched(buf, view), name


def per_column_rel_l2(a, b):
    """Worst relative L2 error over the head-dimension columns."""
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    a, b = a.reshape(-1, a.shape[-1]), b.reshape(-1, b.shape[-1])
    return max(rel_l2(a[:, c], b[:, c]) for c in range(a.shape[1]))


FP16_CASES = [
    # B, H, N, d, causal, padded, p
    (1, 2, 190, 64, True, False, 0.0),
    (2, 2, 333, 128, False, True, 0.1),
    (2, 1, 129, 128, True, True, 0.2),
]


@pytest.mark.parametrize("case", FP16_CASES, ids=lambda c: "B{}H{}N{}d{}{}{}{}".format(
    *c[:4], "-causal" if c[4] else "", "-pad" if c[5] else "", f"-p{c[6]}" if c[6] else ""))
def test_fp16_matches_oracle(case):
    B, H, N, d, causal, padded, p = case
    seed = 0x5151
    note(f"fp16 oracle {case}")
    inp = draw(B, H, N, d, torch.float16, seed=FP16_CASES.index(case) + 300, padded=padded)
    scale = float(np.float32(1 / math.sqrt(d)))
    q, k, v, do = (t.to(DEV) for t in (inp.q, inp.k, inp.v, inp.dout))
    kl = None if inp.key_lens is None else inp.key_lens.to(DEV)
    lens = None if inp.key_lens is None else inp.key_lens.tolist()
    o, lse = binding.forward(q, k, v, scale, causal, kl, p, seed)
    g = binding.backward(q, k, v, o, do, lse, scale, causal, kl, p, seed)
    torch.cuda.synchronize()
    ro, rlse = attention_forward(inp.q, inp.k, inp.v, scale, causal, lens, p, seed)
    eo, el = max_abs(f64(o), ro), max_abs(f64(lse), rlse)
    ref = attention_backward(inp.q, inp.k, inp.v, inp.dout, scale, causal, lens, p, seed)
    errs = [rel_l2(f64(a), b) for a, b in zip(g, ref)]
    cols = [per_column_rel_l2(f64(a), b) for a, b in zip(g, ref)]
    note(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e} relL2 {errs} worst column {cols}")
    assert eo <= TOL_O and el <= TOL_LSE
    assert max(errs) <= TOL_GRAD and max(cols) <= 2 * TOL_GRAD


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
def test_autograd_bnhd_reads_and_writes_in_place(dt, monkeypatch):
    B, N, H, d = 2, 257, 4, 64
    note(f"autograd bnhd in place {dt}")
    g = torch.Generator().manual_seed(77)
    x = [torch.randn(B, N, H, d, generator=g).to(dt).to(DEV) for _ in range(4)]
    seen = {}

    def record(name, fn):
        def wrapped(*args, **kw):
            seen[name] = [t.data_ptr() for t in args if isinstance(t, torch.Tensor)]
            return fn(*args, **kw)
        return wrapped

    monkeypatch.setattr(binding, "fa_fwd_strided", record("fwd", binding.fa_fwd_strided))
    monkeypatch.setattr(binding, "fa_bwd_strided", record("bwd", binding.fa_bwd_strided))
    q, k, v = (t.clone().requires_grad_(True) for t in x[:3])
    o = autograd.flash_attention(q, k, v, causal=True, layout="bnhd")
    o.backward(x[3])
    torch.cuda.synchronize()
    # q, k, v went to the library as views of the caller's memory, and O and
    # the gradients come back in [B, N, H, d] memory
    assert seen["fwd"][:3] == [q.data_ptr(), k.data_ptr(), v.data_ptr()]
    assert seen["bwd"][:3] == [q.data_ptr(), k.data_ptr(), v.data_ptr()]
    assert seen["bwd"][4] == x[3].data_ptr()  # dO read in place too
    assert o.shape == (B, N, H, d) and o.is_contiguous()
    for t in (q, k, v):
        assert t.grad.shape == (B, N, H, d) and t.grad.is_contiguous()
    # the same values as contiguous [B, H, N, d] copies through fa_fwd / fa_bwd
    # (the plain entry points; autograd would take the split forward at this
    # size for contiguous inputs): equal bits
    qc, kc, vc, doc = (t.detach().transpose(1, 2).contiguous() for t in (q, k, v, x[3]))
    oc, lse = binding.forward(qc, kc, vc, d ** -0.5, True)
    gc = binding.backward(qc, kc, vc, oc, doc, lse, d ** -0.5, True)
    torch.cuda.synchronize()
    assert torch.equal(o, oc.transpose(1, 2))
    for t, tc in zip((q, k, v), gc):
        assert torch.equal(t.grad, tc.transpose(1, 2))
