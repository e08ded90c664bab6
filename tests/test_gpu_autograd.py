"""GPU: the torch.autograd entry point (io_aware_exact_24_amd.autograd) against
the fp64 oracle and against the C-ABI calls it wraps."""

import numpy as np
import pytest
import torch

from fa_testlib import TOL_GRAD, TOL_O, f64, max_abs, note, rel_l2
from io_aware_exact_24_amd import binding
from io_aware_exact_24_amd.autograd import flash_attention, scaled_dot_product_attention
from io_aware_exact_24_amd.workloads import draw
from oracle import attention_backward, attention_forward

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def leaf(t, layout):
    t = t.to(DEV)
    if layout == "bnhd":
        t = t.transpose(1, 2).contiguous()
    return t.requires_grad_(True)


@pytest.mark.parametrize("layout", ["bhnd", "bnhd"])
@pytest.mark.parametrize("causal,padded", [(True, False), (False, True)])
def test_autograd_matches_oracle(layout, causal, padded):
    B, H, N, d = 2, 3, 200, 128
    inp = draw(B, H, N, d, torch.bfloat16, seed=77, padded=padded)
    scale = float(np.float32(1 / np.sqrt(d)))
    q, k, v = (leaf(t, layout) for t in (inp.q, inp.k, inp.v))
    do = inp.dout.to(DEV)
    if layout == "bnhd":
        do = do.transpose(1, 2).contiguous()
    o = flash_attention(q, k, v, scale=scale, causal=causal, key_lens=inp.key_lens, layout=layout)
    (o.float() * do.float()).sum().backward()
    torch.cuda.synchronize()
    back = (lambda t: t.transpose(1, 2)) if layout == "bnhd" else (lambda t: t)
    kl = None if inp.key_lens is None else inp.key_lens.tolist()
    ro, _ = attention_forward(inp.q, inp.k, inp.v, scale, causal, kl)
    ref = attention_backward(inp.q, inp.k, inp.v, inp.dout, scale, causal, kl)
    eo = max_abs(f64(back(o)), ro)
    errs = [rel_l2(f64(back(t.grad)), r) for t, r in zip((q, k, v), ref)]
    note(f"{layout} causal={causal} padded={padded}: max|dO|={eo:.2e} relL2={errs}")
    assert eo <= TOL_O and max(errs) <= TOL_GRAD


def test_small_shapes_take_the_split_passes():
    # B*H*blocks below the CU count: the forward and the backward run split (as
    # many shares as split_count / backward_split_count pick); results equal
    # fa_fwd_split's and fa_bwd_split's with those counts bit for bit and the
    # oracle's within the bar
    from io_aware_exact_24_amd.autograd import _bwd_splits, _splits

    B, H, N, d = 1, 2, 1000, 128
    inp = draw(B, H, N, d, torch.bfloat16, seed=80)
    q, k, v = (leaf(t, "bhnd") for t in (inp.q, inp.k, inp.v))
    do = inp.dout.to(DEV)
    s = _splits(q, True)
    assert s >= 2
    o = flash_attention(q, k, v, causal=True)
    sb = _bwd_splits(q, True, (q, k, v, o, do))
    assert sb >= 2
    o.backward(do)
    qd, kd, vd = (t.detach() for t in (q, k, v))
    o2, lse2 = binding.forward_split(qd, kd, vd, d ** -0.5, True, None, 0.0, 0, s)
    g2 = binding.backward_split(qd, kd, vd, o2, do, lse2, d ** -0.5, True, None, 0.0, 0, sb)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for t, g in zip((q, k, v), g2):
        assert torch.equal(t.grad, g)
    ro, _ = attention_forward(inp.q, inp.k, inp.v, float(np.float32(d ** -0.5)), True)
    ref = attention_backward(inp.q, inp.k, inp.v, inp.dout, float(np.float32(d ** -0.5)), True)
    assert max_abs(f64(o), ro) <= TOL_O
    assert max(rel_l2(f64(t.grad), r) for t, r in zip((q, k, v), ref)) <= TOL_GRAD


def test_autograd_equals_c_abi_calls_with_dropout():
    # the Function replays the forward's seed: results are the bits of
    # fa_fwd / fa_bwd called directly with that seed
    B, H, N, d, p, seed = 1, 2, 300, 64, 0.2, 12345
    inp = draw(B, H, N, d, torch.bfloat16, seed=78)
    q, k, v = (leaf(t, "bhnd") for t in (inp.q, inp.k, inp.v))
    do = inp.dout.to(DEV)
    o = flash_attention(q, k, v, causal=True, dropout_p=p, seed=seed)
    o.backward(do)
    qd, kd, vd = (t.detach() for t in (q, k, v))
    from io_aware_exact_24_amd.autograd import _forward

    o2, lse2 = _forward(qd, kd, vd, d ** -0.5, True, None, p, seed)
    g2 = binding.backward(qd, kd, vd, o2, do, lse2, d ** -0.5, True, None, p, seed)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for t, g in zip((q, k, v), g2):
        assert torch.equal(t.grad, g)


def test_sdpa_names_and_no_grad_path():
    B, H, N, d = 2, 2, 130, 64
    inp = draw(B, H, N, d, torch.bfloat16, seed=79)
    q, k, v = (t.to(DEV) for t in (inp.q, inp.k, inp.v))
    with torch.no_grad():
        o = scaled_dot_product_attention(q, k, v, is_causal=True)
    o2 = flash_attention(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    ro, _ = attention_forward(inp.q, inp.k, inp.v, float(np.float32(d ** -0.5)), True)
    assert max_abs(f64(o), ro) <= TOL_O
