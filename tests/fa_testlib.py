"""Shared helpers for the GPU parity tests: run the library on seeded inputs and
compare with the oracle under the stated tolerances."""

import sys

import numpy as np
import torch

from io_aware_exact_24_amd import binding

# Tolerances: dropout masks bit-exact; fp32 max |err| <= 1e-5 on O and LSE;
# bf16 max |err| <= 2e-2 on O, <= 1e-3 on LSE, whole-tensor relative L2 <= 2e-2
# on dQ, dK and dV.
TOL_F32 = 1e-5
TOL_O = 2e-2
TOL_LSE = 1e-3
TOL_GRAD = 2e-2

DEV = "cuda:0"


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(inp):
    kl = None if inp.key_lens is None else inp.key_lens.to(DEV)
    do = None if inp.dout is None else inp.dout.to(DEV)
    return inp.q.to(DEV), inp.k.to(DEV), inp.v.to(DEV), do, kl


def gpu_forward(inp, scale, causal=False, dropout_p=0.0, seed=0):
    q, k, v, _, kl = to_dev(inp)
    o, lse = binding.forward(q, k, v, scale, causal, kl, dropout_p, seed)
    torch.cuda.synchronize()
    return o, lse


def gpu_backward(inp, o, lse, scale, causal=False, dropout_p=0.0, seed=0):
    q, k, v, do, kl = to_dev(inp)
    dq, dk, dv = binding.backward(q, k, v, o, do, lse, scale, causal, kl, dropout_p, seed)
    torch.cuda.synchronize()
    return dq, dk, dv


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def max_abs(a, b):
    a, b = np.asarray(a), np.asarray(b)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):  # -inf - -inf on empty rows, masked here
        d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.max(d)) if d.size else 0.0


def rel_l2(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    if nb == 0.0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


def key_lens_list(inp):
    return None if inp.key_lens is None else inp.key_lens.tolist()
