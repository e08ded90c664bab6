"""Pins for the oracle's analytic backward, independent of the oracle itself.

The gradients are checked against central finite differences of the oracle's
own forward loss sum(dO * O) in fp64 (so a dropped term or a transposed operand
in the closed form shows up), against PyTorch autograd through SDPA in fp64,
and against closed forms: Q = 0, N = 1, and sum_j dK_j = 0 (every row of dS
sums to zero because D_i equals sum_j P_ij dP_ij).
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention_backward, attention_forward, backward_preprocess

RNG = np.random.default_rng(7)


def rand(*shape):
    return RNG.standard_normal(shape)


def _loss(q, k, v, do, **kw):
    o, _ = attention_forward(q, k, v, **kw)
    return float(np.sum(o * do))


@pytest.mark.parametrize("n,d,causal,key_len,p", [
    (1, 1, False, 1, 0.0), (2, 2, False, 2, 0.0), (3, 4, True, 3, 0.0),
    (5, 2, False, 3, 0.0), (5, 4, True, 4, 0.0), (17, 1, True, 17, 0.0),
    (6, 2, False, 6, 0.3), (7, 3, True, 5, 0.25),
])
def test_finite_differences(n, d, causal, key_len, p):
    q, k, v, do = rand(1, 1, n, d), rand(1, 1, n, d), rand(1, 1, n, d), rand(1, 1, n, d)
    kw = dict(scale=0.7, causal=causal, key_lens=[key_len], dropout_p=p, seed=0xABCDEF12345)
    dq, dk, dv = attention_backward(q, k, v, do, **kw)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = _loss(args["q"], args["k"], args["v"], do, **kw)
            args[name] = xm
            fm = _loss(args["q"], args["k"], args["v"], do, **kw)
            num[idx] = (fp - fm) / (2 * h)
        denom = max(1.0, np.abs(num).max())
        assert np.abs(num - g).max() / denom <= 1e-6, name


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd_fp64(causal):
    B, H, N, d = 2, 2, 23, 8
    q, k, v, do = rand(B, H, N, d), rand(B, H, N, d), rand(B, H, N, d), rand(B, H, N, d)
    key_lens = [N, 15]
    scale = 1 / math.sqrt(d)
    dq, dk, dv = attention_backward(q, k, v, do, scale, causal=causal, key_lens=key_lens)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    j = torch.arange(N)
    mask = torch.stack([(j[None, :] < L).expand(N, N) for L in key_lens])[:, None]
    if causal:
        mask = mask & torch.tril(torch.ones(N, N, dtype=torch.bool))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11)


@pytest.mark.parametrize("p", [0.0, 0.2])
def test_key_gradients_sum_to_zero(p):
    q, k, v, do = rand(2, 3, 19, 5), rand(2, 3, 19, 5), rand(2, 3, 19, 5), rand(2, 3, 19, 5)
    _, dk, _ = attention_backward(q, k, v, do, 0.45, causal=True, key_lens=[19, 11],
                                  dropout_p=p, seed=99)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)


def test_zero_queries_value_gradient_closed_form():
    # Q = 0: P_ij = 1/L_i on allowed keys, so dV_j = sum over rows i that allow j of dO_i / L_i.
    N, d = 11, 3
    do = rand(1, 1, N, d)
    for causal, L in [(False, N), (True, N), (True, 7), (False, 4)]:
        _, _, dv = attention_backward(np.zeros((1, 1, N, d)), rand(1, 1, N, d), rand(1, 1, N, d),
                                      do, 0.9, causal=causal, key_lens=[L])
        for j in range(N):
            ref = np.zeros(d)
            for i in range(N):
                cnt = min(L, i + 1) if causal else L
                if j < cnt:
                    ref += do[0, 0, i] / cnt
            np.testing.assert_allclose(dv[0, 0, j], ref, atol=1e-14)


def test_single_token():
    q, k, v, do = rand(2, 2, 1, 4), rand(2, 2, 1, 4), rand(2, 2, 1, 4), rand(2, 2, 1, 4)
    dq, dk, dv = attention_backward(q, k, v, do, 0.5)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)
    np.testing.assert_array_equal(dv, do)


def test_empty_rows_have_zero_gradient():
    q, k, v, do = rand(1, 1, 6, 2), rand(1, 1, 6, 2), rand(1, 1, 6, 2), rand(1, 1, 6, 2)
    dq, dk, dv = attention_backward(q, k, v, do, 0.5, key_lens=[0])
    assert np.all(dq == 0) and np.all(dk == 0) and np.all(dv == 0)


def test_selected_rows_agree_with_whole():
    B, H, N, d = 1, 2, 33, 4
    q, k, v, do = rand(B, H, N, d), rand(B, H, N, d), rand(B, H, N, d), rand(B, H, N, d)
    kw = dict(scale=0.5, causal=True, dropout_p=0.1, seed=5)
    dq, dk, dv = attention_backward(q, k, v, do, **kw)
    rows = np.array([0, 3, 32])
    dq2, dk2, dv2 = attention_backward(q, k, v, do, q_rows=rows, k_rows=rows, row_chunk=5, **kw)
    np.testing.assert_allclose(dq2, dq[:, :, rows], atol=1e-13)
    np.testing.assert_allclose(dk2, dk[:, :, rows], atol=1e-13)
    np.testing.assert_allclose(dv2, dv[:, :, rows], atol=1e-13)
    dq3, _, _ = attention_backward(q, k, v, do, q_rows=rows, k_rows=[], **kw)
    np.testing.assert_allclose(dq3, dq[:, :, rows], atol=1e-13)


def test_preprocess_term_equals_jacobian_contraction():
    # D_i = sum_k dO_ik O_ik must equal sum_j P_ij dP_ij with dP = dO V^T (p = 0).
    N, d = 9, 3
    q, k, v, do = rand(1, 1, N, d), rand(1, 1, N, d), rand(1, 1, N, d), rand(1, 1, N, d)
    o, _ = attention_forward(q, k, v, 0.8)
    V = np.eye(N)[None, None]
    pad = ((0, 0), (0, 0), (0, 0), (0, N - d))
    p, _ = attention_forward(np.pad(q, pad), np.pad(k, pad), V, 0.8)
    dp = do[0, 0] @ v[0, 0].T
    np.testing.assert_allclose(backward_preprocess(o, do)[0, 0], np.sum(p[0, 0] * dp, axis=1),
                               atol=1e-13)


def test_first_row_restriction_is_exact_for_causal():
    B, H, N, d = 1, 1, 40, 4
    q, k, v, do = rand(B, H, N, d), rand(B, H, N, d), rand(B, H, N, d), rand(B, H, N, d)
    kw = dict(scale=0.6, causal=True)
    dq, dk, dv = attention_backward(q, k, v, do, **kw)
    keys, rows = np.array([25, 30, 39]), np.array([3, 26])
    dq2, dk2, dv2 = attention_backward(q, k, v, do, q_rows=rows, k_rows=keys, first_row=25, **kw)
    np.testing.assert_allclose(dk2, dk[:, :, keys], atol=1e-13)
    np.testing.assert_allclose(dv2, dv[:, :, keys], atol=1e-13)
    np.testing.assert_allclose(dq2, dq[:, :, rows], atol=1e-13)
    with pytest.raises(ValueError):
        attention_backward(q, k, v, do, q_rows=rows, k_rows=keys, first_row=26, **kw)
