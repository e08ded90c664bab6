"""Pins for the oracle's forward pass, independent of the oracle itself.

Each check comes from the mathematics of softmax attention or from an
independent implementation: pure-Python loops over the definition, PyTorch's
scaled_dot_product_attention in fp64 (ML Canon 48 FlashAttention, the PyTorch
SDPA box, states it computes softmax(QK^T/sqrt(d))V), closed forms (Q = 0,
constant V, identical keys, causal row 0) and symmetries (key shift, key/value
permutation).  A deliberately wrong tiled sketch must be rejected by the same
comparison the GPU tests use.
"""

import math

import numpy as np
import pytest
import torch

from oracle import allowed_mask, attention_forward

RNG = np.random.default_rng(20261202)


def rand(*shape):
    return RNG.standard_normal(shape)


def brute_forward_head(q, k, v, scale, causal, key_len):
    """The definition with Python loops and the math module (no numpy arithmetic)."""
    n, d = len(q), len(q[0])
    out = [[0.0] * d for _ in range(n)]
    lse = [0.0] * n
    for i in range(n):
        scores = []
        for j in range(n):
            if j < key_len and (not causal or j <= i):
                scores.append((j, scale * math.fsum(q[i][t] * k[j][t] for t in range(d))))
        if not scores:
            lse[i] = -math.inf
            continue
        m = max(s for _, s in scores)
        den = math.fsum(math.exp(s - m) for _, s in scores)
        lse[i] = m + math.log(den)
        for t in range(d):
            out[i][t] = math.fsum(math.exp(s - m) / den * v[j][t] for j, s in scores)
    return out, lse


@pytest.mark.parametrize("n,d,causal,key_len", [
    (1, 3, False, 1), (5, 2, False, 5), (7, 3, True, 7), (8, 4, False, 5),
    (6, 2, True, 4), (9, 1, True, 9), (4, 3, False, 0), (5, 2, True, 0),
])
def test_matches_python_loops(n, d, causal, key_len):
    q, k, v = rand(1, 1, n, d), rand(1, 1, n, d), rand(1, 1, n, d)
    scale = 0.37
    o, lse = attention_forward(q, k, v, scale, causal=causal, key_lens=[key_len])
    bo, blse = brute_forward_head(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(),
                                  scale, causal, key_len)
    np.testing.assert_allclose(o[0, 0], np.array(bo), rtol=0, atol=1e-13)
    np.testing.assert_array_equal(np.isinf(lse[0, 0]), np.isinf(np.array(blse)))
    fin = np.isfinite(np.array(blse))
    np.testing.assert_allclose(lse[0, 0][fin], np.array(blse)[fin], rtol=0, atol=1e-13)


def _sdpa_mask(B, N, causal, key_lens):
    m = torch.ones(B, 1, N, N, dtype=torch.bool)
    j = torch.arange(N)
    for b in range(B):
        L = N if key_lens is None else key_lens[b]
        m[b, 0] &= (j[None, :] < L)
    if causal:
        m &= torch.tril(torch.ones(N, N, dtype=torch.bool))
    return m


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
def test_matches_torch_sdpa_fp64(causal, padded):
    B, H, N, d = 2, 3, 37, 16
    q, k, v = rand(B, H, N, d), rand(B, H, N, d), rand(B, H, N, d)
    key_lens = [N - 5, 11] if padded else None
    scale = 1.0 / math.sqrt(d)
    o, _ = attention_forward(q, k, v, scale, causal=causal, key_lens=key_lens)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    mask = _sdpa_mask(B, N, causal, key_lens)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)


def test_probabilities_rows_sum_to_one():
    # With V = identity (d = N) the output row i is the probability row P_i.
    N = 12
    q, k = rand(1, 1, N, 5), rand(1, 1, N, 5)
    v = np.eye(N)[None, None]
    for causal, L in [(False, N), (True, N), (False, 7), (True, 3)]:
        p, _ = attention_forward(np.pad(q, ((0, 0), (0, 0), (0, 0), (0, N - 5))),
                                 np.pad(k, ((0, 0), (0, 0), (0, 0), (0, N - 5))), v, 0.8,
                                 causal=causal, key_lens=[L])
        ok = allowed_mask(np.arange(N), N, causal, L)
        rows = ok.any(axis=1)
        np.testing.assert_allclose(p[0, 0].sum(axis=1)[rows], 1.0, atol=1e-14)
        assert np.all(p[0, 0][~ok] == 0.0)
        assert np.all(p[0, 0] >= 0.0)


def test_constant_v_returns_v():
    N, d = 20, 6
    c = rand(d)
    v = np.broadcast_to(c, (1, 1, N, d)).copy()
    o, _ = attention_forward(rand(1, 1, N, d), rand(1, 1, N, d), v, 0.5, causal=True)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(c, (N, d)), atol=1e-14)


def test_identical_keys_average_allowed_values():
    N, d = 10, 4
    k = np.broadcast_to(rand(d), (1, 1, N, d)).copy()
    v = rand(1, 1, N, d)
    for causal, L in [(False, N), (True, N), (False, 6)]:
        o, _ = attention_forward(rand(1, 1, N, d), k, v, 0.9, causal=causal, key_lens=[L])
        for i in range(N):
            hi = min(L, i + 1) if causal else L
            np.testing.assert_allclose(o[0, 0, i], v[0, 0, :hi].mean(axis=0), atol=1e-14)


def test_causal_row_zero_is_v0():
    o, lse = attention_forward(rand(2, 2, 9, 3), rand(2, 2, 9, 3), v := rand(2, 2, 9, 3),
                               1.3, causal=True)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])


def test_zero_queries_closed_form():
    # Q = 0: every allowed score is 0, P_i is uniform over the L_i allowed keys,
    # LSE_i = ln(L_i) and O_i is the mean of the allowed values.
    N, d = 16, 3
    v = rand(1, 1, N, d)
    for causal, L in [(False, N), (True, N), (True, 10), (False, 5)]:
        o, lse = attention_forward(np.zeros((1, 1, N, d)), rand(1, 1, N, d), v, 0.7,
                                   causal=causal, key_lens=[L])
        for i in range(N):
            cnt = min(L, i + 1) if causal else L
            assert lse[0, 0, i] == pytest.approx(math.log(cnt), abs=1e-14)
            np.testing.assert_allclose(o[0, 0, i], v[0, 0, :cnt].mean(axis=0), atol=1e-14)


def test_key_shift_invariance():
    # K -> K + u (same u for every key) adds scale*q_i.u to every score of row i:
    # O is unchanged and LSE_i moves by exactly that amount.
    N, d, scale = 15, 5, 0.6
    q, k, v = rand(1, 1, N, d), rand(1, 1, N, d), rand(1, 1, N, d)
    u = rand(d)
    o1, l1 = attention_forward(q, k, v, scale, causal=True, key_lens=[12])
    o2, l2 = attention_forward(q, k + u, v, scale, causal=True, key_lens=[12])
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, scale * (q @ u), atol=1e-12)


def test_joint_key_value_permutation_invariance():
    N, d = 14, 4
    q, k, v = rand(1, 1, N, d), rand(1, 1, N, d), rand(1, 1, N, d)
    perm = RNG.permutation(N)
    o1, l1 = attention_forward(q, k, v, 0.5)
    o2, l2 = attention_forward(q, k[:, :, perm], v[:, :, perm], 0.5)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_single_key_returns_value():
    q, k, v = rand(3, 2, 1, 8), rand(3, 2, 1, 8), rand(3, 2, 1, 8)
    o, lse = attention_forward(q, k, v, 0.25)
    np.testing.assert_array_equal(o, v)
    np.testing.assert_allclose(lse[..., 0], 0.25 * np.sum(q * k, axis=-1)[..., 0], atol=1e-14)


def test_lse_bounds():
    N, d, scale = 30, 6, 0.4
    q, k, v = rand(1, 1, N, d), rand(1, 1, N, d), rand(1, 1, N, d)
    _, lse = attention_forward(q, k, v, scale, causal=True)
    s = scale * q[0, 0] @ k[0, 0].T
    for i in range(N):
        mx = s[i, : i + 1].max()
        assert mx - 1e-12 <= lse[0, 0, i] <= mx + math.log(i + 1) + 1e-12


def test_rows_and_chunks_agree_with_whole():
    N, d = 40, 8
    q, k, v = rand(2, 2, N, d), rand(2, 2, N, d), rand(2, 2, N, d)
    o, lse = attention_forward(q, k, v, 0.3, causal=True, key_lens=[33, 40])
    rows = np.array([0, 5, 17, 39])
    o2, l2 = attention_forward(q, k, v, 0.3, causal=True, key_lens=[33, 40], rows=rows, row_chunk=3)
    np.testing.assert_allclose(o2, o[:, :, rows], atol=1e-14)
    np.testing.assert_allclose(l2, lse[:, :, rows], atol=1e-14)


def _tiled_sketch_without_rescale(q, k, v, scale, tile):
    """Negative control: the tiling shortcut of the hardware-aware page (section
    2.1), which normalises each key tile on its own and adds the tiles'
    outputs with no running max or rescale.  Written here as one blockwise
    softmax: the score matrix is viewed as [n/t, t, n/t, t] blocks, each
    (query block, key block) pair is softmax-normalised over its own t keys,
    and the block outputs are summed over the key-block axis.  The weights of
    a row then sum to the number of key blocks, so the result is exact only
    when there is one key block.  n must be a multiple of t."""
    n, dv = q.shape[0], v.shape[1]
    nb = n // tile
    s = (scale * q @ k.T).reshape(nb, tile, nb, tile)
    e = np.exp(s - s.max(axis=3, keepdims=True))
    w = e / e.sum(axis=3, keepdims=True)
    return np.einsum("aibj,bjc->aic", w, v.reshape(nb, tile, dv)).reshape(n, dv)


@pytest.mark.parametrize("n,tile,should_pass", [(64, 64, True), (128, 64, False), (96, 32, False)])
def test_negative_control_tiled_sketch(n, tile, should_pass):
    q, k, v = rand(n, 16), rand(n, 16), rand(n, 16)
    ref, _ = attention_forward(q[None, None], k[None, None], v[None, None], 0.25)
    bad = _tiled_sketch_without_rescale(q, k, v, 0.25, tile)
    err = np.abs(bad - ref[0, 0]).max()
    assert (err <= 2e-2) == should_pass


def test_dropout_scale_closed_form():
    # Q = 0 and V = ones: O_i = (number of kept allowed keys) * s / L_i with
    # s = fp32(1/(1-p)), the inverted-dropout scale.
    from oracle import keep_mask

    N, p, seed = 64, 0.3, 0x77
    v = np.ones((1, 1, N, 1))
    o, lse = attention_forward(np.zeros((1, 1, N, 1)), rand(1, 1, N, 1), v, 1.0,
                               causal=True, dropout_p=p, seed=seed)
    keep = keep_mask(seed, 0, 0, np.arange(N), np.arange(N), p)
    s = float(np.float32(1.0 / (1.0 - float(np.float32(p)))))
    for i in range(N):
        kept = int(keep[i, : i + 1].sum())
        assert o[0, 0, i, 0] == pytest.approx(kept * s / (i + 1), abs=1e-14)
        # LSE is the normaliser before dropout
        assert lse[0, 0, i] == pytest.approx(math.log(i + 1), abs=1e-14)
