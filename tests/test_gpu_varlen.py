"""GPU tests of packed variable-length batches (fa_fwd_varlen, fa_bwd_varlen).

Sequence b of a packed batch is the same attention as entry b of a padded
batch whose key lengths are the sequence lengths, restricted to its first
len_b query rows, and with dO zero on the padded query rows (which then add
nothing to dK and dV).  The packed results must equal the padded ones bit for
bit (the same kernels over the same tiles; the extra padded tiles only add
zeros), and the oracle's within the tolerances.
"""

import math

import numpy as np
import pytest
import torch

from fa_testlib import DEV, TOL_GRAD, TOL_LSE, TOL_O, f64, max_abs, note, rel_l2
from io_aware_exact_24_amd import binding
from oracle import attention_backward, attention_forward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


LENS = [77, 0, 1, 300, 128, 33]


@pytest.mark.parametrize("dt,d,causal,p", [
    (torch.bfloat16, 64, True, 0.0),
    (torch.bfloat16, 128, False, 0.1),
    (torch.float16, 64, False, 0.0),
    (torch.bfloat16, 96, True, 0.1),    # the generic kernels
    (torch.float32, 64, True, 0.0),
], ids=lambda x: str(x).replace("torch.", ""))
def test_varlen_equals_padded_and_oracle(dt, d, causal, p):
    H, seed = 3, 0xABCDEF
    B, L = len(LENS), max(LENS)
    cu = np.concatenate([[0], np.cumsum(LENS)]).astype(np.int32)
    T = int(cu[-1])
    note(f"varlen {dt} d={d} causal={causal} p={p} lens={LENS}")
    g = torch.Generator().manual_seed(d + int(causal))
    # padded [B, H, L, d] inputs; dO zero past each length
    pad = [torch.randn(B, H, L, d, generator=g).to(dt) for _ in range(4)]
    for b, n in enumerate(LENS):
        for t in pad:
            t[b, :, n:] = 0
    # packed [T, H, d] copies of the valid rows
    packed = [torch.cat([t[b, :, :n].transpose(0, 1) for b, n in enumerate(LENS)]) for t in pad]
    q, k, v, do = (t.to(DEV) for t in packed)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = binding.forward_varlen(q, k, v, cu, scale, causal, p, seed)
    dq, dk, dv = binding.backward_varlen(q, k, v, o, do, lse, cu, scale, causal, p, seed)
    # the padded batch on the same kernels
    kl = torch.tensor(LENS, dtype=torch.int32, device=DEV)
    qp, kp, vp, dop = (t.to(DEV) for t in pad)
    op, lsep = binding.forward(qp, kp, vp, scale, causal, kl, p, seed)
    gp = binding.backward(qp, kp, vp, op, dop, lsep, scale, causal, kl, p, seed)
    torch.cuda.synchronize()
    for b, n in enumerate(LENS):
        t0 = int(cu[b])
        assert torch.equal(o[t0:t0 + n], op[b, :, :n].transpose(0, 1)), b
        assert torch.equal(lse[H * t0:H * (t0 + n)].view(H, n), lsep[b, :, :n]), b
        for name, a, r in (("dq", dq, gp[0]), ("dk", dk, gp[1]), ("dv", dv, gp[2])):
            assert torch.equal(a[t0:t0 + n], r[b, :, :n].transpose(0, 1)), (name, b)
    # and the oracle on the padded form
    lens = list(LENS)
    ro, rlse = attention_forward(pad[0], pad[1], pad[2], scale, causal, lens, p, seed)
    rg = attention_backward(pad[0], pad[1], pad[2], pad[3], scale, causal, lens, p, seed)
    # the oracle's padded rows, packed like the GPU's (token-major [T, H, d])
    def pack(r):
        return np.concatenate([r[b, :, :n].transpose(1, 0, 2) for b, n in enumerate(LENS)])
    eo = max_abs(f64(o), pack(ro))
    el = max_abs(f64(lse), np.concatenate([rlse[b, :, :n].reshape(-1) for b, n in enumerate(LENS)]))
    # whole-tensor relative L2 over all tokens, and the worst head-dimension
    # column (a one-token sequence has exactly zero dQ and dK, so a relative
    # error per sequence would be meaningless there)
    errs = [rel_l2(f64(a), pack(r)) for a, r in zip((dq, dk, dv), rg)]
    cols = [max(rel_l2(f64(a)[..., c].reshape(-1), pack(r)[..., c].reshape(-1)) for c in range(d))
            for a, r in zip((dq, dk, dv), rg)]
    note(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e} relL2 {errs} worst column {max(cols):.3e}")
    if dt == torch.float32:
        assert eo <= 1e-5 and el <= 1e-5 and max(errs) <= 1e-5 and max(cols) <= 2e-5
    else:
        assert eo <= TOL_O and el <= TOL_LSE and max(errs) <= TOL_GRAD and max(cols) <= 2 * TOL_GRAD


def test_varlen_reads_qkv_in_place():
    # q, k, v as views of one fused [T, 3, H, d] projection buffer
    lens, H, d = [50, 200, 3], 2, 128
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    note(f"varlen fused qkv lens={lens}")
    g = torch.Generator().manual_seed(5)
    qkv = torch.randn(T, 3, H, d, generator=g).to(torch.bfloat16).to(DEV)
    q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    scale = d ** -0.5
    o, lse = binding.forward_varlen(q, k, v, cu, scale, True)
    oc, lsec = binding.forward_varlen(q.contiguous(), k.contiguous(), v.contiguous(), cu, scale, True)
    torch.cuda.synchronize()
    assert torch.equal(o, oc) and torch.equal(lse, lsec)


@pytest.mark.parametrize("dt,d,causal,p,max_len", [
    (torch.bfloat16, 64, True, 0.0, 300),
    (torch.bfloat16, 128, False, 0.1, 300),
    (torch.float16, 64, False, 0.0, 512),     # max_len above the longest sequence
    (torch.bfloat16, 96, True, 0.1, 300),     # padded head size
    (torch.float16, 32, False, 0.2, 300),     # padded head size
    (torch.bfloat16, 128, True, 0.0, 301),
], ids=lambda x: str(x).replace("torch.", ""))
def test_varlen_device_offsets_equal_host_offsets(dt, d, causal, p, max_len):
    # One launch over every sequence (offsets on the device) against one
    # launch per sequence (host offsets): the same tiles of the same kernels,
    # so every output must be equal bit for bit.
    H, seed = 3, 0x5EED5
    cu = np.concatenate([[0], np.cumsum(LENS)]).astype(np.int32)
    T = int(cu[-1])
    note(f"varlen device offsets {dt} d={d} causal={causal} p={p} max_len={max_len} lens={LENS}")
    g = torch.Generator().manual_seed(d + 7)
    q, k, v, do = (torch.randn(T, H, d, generator=g).to(dt).to(DEV) for _ in range(4))
    scale = float(np.float32(1 / math.sqrt(d)))
    cud = torch.tensor(cu, dtype=torch.int32, device=DEV)
    o1, lse1 = binding.forward_varlen(q, k, v, cu, scale, causal, p, seed)
    g1 = binding.backward_varlen(q, k, v, o1, do, lse1, cu, scale, causal, p, seed)
    o2, lse2 = binding.forward_varlen_device(q, k, v, cud, max_len, scale, causal, p, seed)
    g2 = binding.backward_varlen_device(q, k, v, o1, do, lse1, cud, max_len, scale, causal, p, seed)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(lse1, lse2)
    for name, a, b in zip(("dq", "dk", "dv"), g1, g2):
        assert torch.equal(a, b), name


def test_varlen_device_many_sequences():
    # 200 sequences of 1 .. 200 tokens in one launch per pass, against the
    # oracle on a few of them
    rng = np.random.default_rng(12)
    lens = rng.integers(1, 201, 200)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, d = int(cu[-1]), 2, 64
    note(f"varlen device offsets, {len(lens)} sequences, {T} tokens")
    g = torch.Generator().manual_seed(13)
    q, k, v, do = (torch.randn(T, H, d, generator=g).to(torch.bfloat16) for _ in range(4))
    scale = float(np.float32(1 / math.sqrt(d)))
    cud = torch.tensor(cu, dtype=torch.int32, device=DEV)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = binding.forward_varlen_device(qd, kd, vd, cud, int(lens.max()), scale, True)
    dq, dk, dv = binding.backward_varlen_device(qd, kd, vd, o, dod, lse, cud, int(lens.max()),
                                                scale, True)
    torch.cuda.synchronize()
    for b in (0, 57, 199, int(np.argmax(lens))):
        t0, n = int(cu[b]), int(lens[b])
        seq = [t[t0:t0 + n].transpose(0, 1)[None] for t in (q, k, v, do)]
        ro, rlse = attention_forward(seq[0], seq[1], seq[2], scale, True)
        rg = attention_backward(seq[0], seq[1], seq[2], seq[3], scale, True)
        eo = max_abs(f64(o[t0:t0 + n].transpose(0, 1))[None], ro)
        el = max_abs(f64(lse[H * t0:H * (t0 + n)]).reshape(1, H, n), rlse)
        errs = [rel_l2(f64(a[t0:t0 + n].transpose(0, 1))[None], r) for a, r in zip((dq, dk, dv), rg)]
        note(f"  sequence {b} (n={n}): max|dO|={eo:.2e} max|dLSE|={el:.2e} relL2 {max(errs):.2e}")
        assert eo <= TOL_O and el <= TOL_LSE
        if n > 1:  # a one-token sequence has exactly zero dQ and dK
            assert max(errs) <= TOL_GRAD
