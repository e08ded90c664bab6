"""GPU: the split-KV forward (fa_fwd_split) against the fp64 oracle and
against fa_fwd on the same inputs."""

import numpy as np
import pytest
import torch

from fa_testlib import TOL_LSE, TOL_O, f64, gpu_forward, key_lens_list, max_abs, note
from io_aware_exact_24_amd import binding
from io_aware_exact_24_amd.workloads import Inputs, draw
from oracle import attention_forward

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


CASES = [
    # B, H, N, d, causal, key lengths ("draw": uniform in [N/4, N]), dropout p, splits
    (1, 2, 1000, 128, True, None, 0.0, 3),
    (2, 1, 513, 64, False, "draw", 0.0, 4),
    (1, 2, 300, 128, True, None, 0.1, 2),
    (1, 1, 100, 64, False, None, 0.0, 5),      # more splits than key tiles
    (2, 2, 700, 128, True, [0, 650], 0.0, 7),  # an empty batch entry
    (1, 1, 64, 128, True, None, 0.0, 1),
    (1, 3, 2048, 64, True, None, 0.2, 16),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}N{}d{}{}-S{}{}".format(
    c[0], c[1], c[2], c[3], "-causal" if c[4] else "", c[7], f"-p{c[6]}" if c[6] else ""))
def test_split_forward(case):
    B, H, N, d, causal, lens, p, S = case
    inp = draw(B, H, N, d, torch.bfloat16, seed=CASES.index(case) + 300, padded=lens == "draw")
    if isinstance(lens, list):
        inp = Inputs(inp.q, inp.k, inp.v, inp.dout, torch.tensor(lens, dtype=torch.int32))
    scale, seed = float(np.float32(1 / np.sqrt(d))), 0x0123456789ABCDEF
    q, k, v = (t.to(DEV) for t in (inp.q, inp.k, inp.v))
    kl = None if inp.key_lens is None else inp.key_lens.to(DEV)
    note(f"split case {case}")
    o, lse = binding.forward_split(q, k, v, scale, causal, kl, p, seed, S)
    torch.cuda.synchronize()
    ro, rlse = attention_forward(inp.q, inp.k, inp.v, scale, causal, key_lens_list(inp), p, seed)
    eo, el = max_abs(f64(o), ro), max_abs(f64(lse), rlse)
    o1, lse1 = gpu_forward(inp, scale, causal, p, seed)
    d1 = max_abs(f64(o), f64(o1))
    note(f"  vs oracle: max|dO|={eo:.2e} max|dLSE|={el:.2e}; vs fa_fwd: max|dO|={d1:.2e}")
    assert eo <= TOL_O and el <= TOL_LSE
    assert np.array_equal(np.isneginf(f64(lse)), np.isneginf(rlse))
    assert d1 <= TOL_O
