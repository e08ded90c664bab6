"""GPU parity of head sizes 32, 96 and 256 in every type, and of the fp32
backward (also at 64 and 128), against the fp64 oracle.  16-bit d = 32 and 96
run on the MFMA kernels of width 64 and 128 with the head dimension
zero-padded on chip; d = 256 and every fp32 case run on the generic kernels.

Tolerances: 16-bit types as everywhere (O max |err| <= 2e-2, LSE <= 1e-3,
gradients whole-tensor relative L2 <= 2e-2 and worst head-dimension column
<= 4e-2); fp32 O and LSE max |err| <= 1e-5.  fp32 gradients: relative L2
<= 1e-5 and worst column <= 2e-5.  Each gradient element is a sum of about N
fp32 products of terms rounded to fp32 (2^-24 relative), so its relative
error grows like sqrt(N) * 2^-24, about 1e-6 at these sizes.
"""

import math

import numpy as np
import pytest
import torch

from fa_testlib import DEV, TOL_F32, TOL_GRAD, TOL_LSE, TOL_O, f64, max_abs, note, rel_l2
from io_aware_exact_24_amd import binding
from io_aware_exact_24_amd.workloads import WORKLOADS, draw, draw_workload
from oracle import attention_backward, attention_forward

pytestmark = pytest.mark.gpu

TOL_GRAD_F32 = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def worst_column(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    a, b = a.reshape(-1, a.shape[-1]), b.reshape(-1, b.shape[-1])
    return max(rel_l2(a[:, c], b[:, c]) for c in range(a.shape[1]))


def run_and_check(B, H, N, d, dt, causal, padded, p, seed, what):
    inp = draw(B, H, N, d, dt, seed=seed, padded=padded)
    scale = float(np.float32(1 / math.sqrt(d)))
    q, k, v, do = (t.to(DEV) for t in (inp.q, inp.k, inp.v, inp.dout))
    kl = None if inp.key_lens is None else inp.key_lens.to(DEV)
    lens = None if inp.key_lens is None else inp.key_lens.tolist()
    dseed = 0x0123456789ABCDEF
    o, lse = binding.forward(q, k, v, scale, causal, kl, p, dseed)
    g = binding.backward(q, k, v, o, do, lse, scale, causal, kl, p, dseed)
    torch.cuda.synchronize()
    ro, rlse = attention_forward(inp.q, inp.k, inp.v, scale, causal, lens, p, dseed)
    ref = attention_backward(inp.q, inp.k, inp.v, inp.dout, scale, causal, lens, p, dseed)
    eo, el = max_abs(f64(o), ro), max_abs(f64(lse), rlse)
    errs = [rel_l2(f64(a), b) for a, b in zip(g, ref)]
    cols = [worst_column(f64(a), b) for a, b in zip(g, ref)]
    note(f"{what}: max|dO|={eo:.3e} max|dLSE|={el:.3e} relL2 dQ={errs[0]:.3e} dK={errs[1]:.3e} "
         f"dV={errs[2]:.3e} worst column {max(cols):.3e}")
    assert np.array_equal(np.isneginf(f64(lse)), np.isneginf(rlse))
    if dt == torch.float32:
        assert eo <= TOL_F32 and el <= TOL_F32, (eo, el)
        assert max(errs) <= TOL_GRAD_F32 and max(cols) <= 2 * TOL_GRAD_F32, (errs, cols)
    else:
        assert eo <= TOL_O and el <= TOL_LSE, (eo, el)
        assert max(errs) <= TOL_GRAD and max(cols) <= 2 * TOL_GRAD, (errs, cols)
    return o, lse, g


TYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}
MASKS = [
    # causal, padded, p  (fp32 takes no dropout)
    (False, False, 0.0),
    (True, True, 0.0),
    (True, False, 0.1),
    (False, True, 0.2),
]


@pytest.mark.parametrize("mask", MASKS, ids=lambda m: "{}{}{}".format(
    "causal" if m[0] else "full", "-pad" if m[1] else "", f"-p{m[2]}" if m[2] else ""))
@pytest.mark.parametrize("d", [32, 96, 256])
@pytest.mark.parametrize("tname", list(TYPES))
def test_generic_head_sizes_match_oracle(tname, d, mask):
    causal, padded, p = mask
    if tname == "f32" and p > 0:
        pytest.skip("fp32 takes no dropout (FA_ERR_UNSUPPORTED)")
    B, H, N = (2, 2, 77) if d == 256 else (2, 3, 130)
    what = f"generic {tname} d={d} B{B} H{H} N{N} causal={causal} padded={padded} p={p}"
    note(what)
    run_and_check(B, H, N, d, TYPES[tname], causal, padded, p, seed=d + MASKS.index(mask), what=what)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,padded", [(False, False), (True, True)])
def test_fp32_backward_matches_oracle(d, causal, padded):
    what = f"fp32 backward d={d} causal={causal} padded={padded}"
    note(what)
    run_and_check(2, 2, 200, d, torch.float32, causal, padded, 0.0, seed=500 + d, what=what)


def test_workload_single_head_fp32_backward():
    # the single-head fp32 workload (B=H=1, N=128, d=64), forward and backward
    w = WORKLOADS[1]
    inp = draw_workload(w)
    note("single_head_fp32 forward + backward")
    q, k, v, do = (t.to(DEV) for t in (inp.q, inp.k, inp.v, inp.dout if inp.dout is not None
                                                              else torch.randn_like(inp.q)))
    o, lse = binding.forward(q, k, v, w.scale, False)
    g = binding.backward(q, k, v, o, do, lse, w.scale, False)
    torch.cuda.synchronize()
    ref = attention_backward(inp.q, inp.k, inp.v, do.cpu(), w.scale, False)
    errs = [max_abs(f64(a), b) for a, b in zip(g, ref)]
    note(f"  max|err| dQ={errs[0]:.3e} dK={errs[1]:.3e} dV={errs[2]:.3e}")
    assert max(errs) <= TOL_F32, errs


@pytest.mark.parametrize("tname,d", [("f32", 64), ("bf16", 96), ("fp16", 256)])
def test_generic_stages_equal_fa_bwd_and_are_repeatable(tname, d):
    dt = TYPES[tname]
    B, H, N = 2, 2, 100
    note(f"generic stages {tname} d={d}")
    inp = draw(B, H, N, d, dt, seed=d, padded=True)
    scale = float(np.float32(1 / math.sqrt(d)))
    q, k, v, do = (t.to(DEV) for t in (inp.q, inp.k, inp.v, inp.dout))
    kl = inp.key_lens.to(DEV)
    p = 0.0 if dt == torch.float32 else 0.1
    o, lse = binding.forward(q, k, v, scale, True, kl, p, 7)
    g1 = binding.backward(q, k, v, o, do, lse, scale, True, kl, p, 7)
    g2 = binding.backward(q, k, v, o, do, lse, scale, True, kl, p, 7)
    ws = torch.empty(binding.fa_bwd_workspace_size(B, H, N, d, binding._dtype_code(q)),
                     dtype=torch.uint8, device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    binding.fa_bwd_dq(q, k, v, o, do, lse, dq, scale, True, kl, p, 7, ws)
    binding.fa_bwd_dkdv(q, k, v, do, dk, dv, scale, True, kl, p, 7, ws)
    torch.cuda.synchronize()
    for a, b, c in zip(g1, g2, (dq, dk, dv)):
        assert torch.equal(a, b) and torch.equal(a, c)


def test_generic_strided_equals_contiguous():
    B, H, N, d = 2, 3, 90, 96
    note("generic strided d=96 [B, N, H, d]")
    inp = draw(B, H, N, d, torch.bfloat16, seed=11, padded=True)
    scale = float(np.float32(1 / math.sqrt(d)))
    q, k, v, do = (t.to(DEV) for t in (inp.q, inp.k, inp.v, inp.dout))
    kl = inp.key_lens.to(DEV)
    o, lse = binding.forward(q, k, v, scale, True, kl, 0.1, 3)
    g = binding.backward(q, k, v, o, do, lse, scale, True, kl, 0.1, 3)
    qs, ks, vs, dos = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v, do))
    os_, lse_s = binding.forward(qs, ks, vs, scale, True, kl, 0.1, 3)
    gs = binding.backward(qs, ks, vs, os_, dos, lse_s, scale, True, kl, 0.1, 3)
    torch.cuda.synchronize()
    assert not os_.is_contiguous()  # the strided entry points ran
    assert torch.equal(os_, o) and torch.equal(lse_s, lse)
    for a, b in zip(gs, g):
        assert torch.equal(a, b)
