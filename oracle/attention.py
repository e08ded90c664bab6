"""Plain fp64 softmax attention, forward and analytic backward.

TEST INFRASTRUCTURE ONLY.  This is the CPU oracle the GPU library is checked
against.  Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import it; the library and its Python binding never do, and this
package imports nothing from them.

What is computed, and where the pages fix it:

* One head of attention is O = Dropout(softmax(mask(scale * Q K^T))) V, with the
  operations in the order product, scale, mask, softmax, dropout, product
  (FlashAttention first principles, section 2 and section 3.2); masking and
  dropout are optional and element-wise (same page, section 4.1).  Heads are independent
  (same page, section 2), so a [B, H, N, d] batch is B*H independent problems.
* The default scale is 1/sqrt(d) (ML Canon 48 FlashAttention, the PyTorch SDPA
  box); here the caller passes it.
* Softmax runs along each row of the N x N score matrix (FlashAttention first
  principles, section 4.2).  The tiled method returns exactly this result
  (ML Canon 48 FlashAttention, "the gist" and "tiling and online softmax"), so
  the oracle is the untiled definition: the whole score matrix of a head is
  materialised in fp64.
* The backward of the tiled method recomputes the probabilities from Q, K and
  the saved row normalisers (ML Canon 48 FlashAttention, "backward without
  N x N"; Flash Attention hardware-aware optimisation, section 2.2).  Its values are
  the gradients of the definition above, written here in closed form.

Readings where the pages are silent (all fixed here and used by both sides):

* mask(i, j) keeps key j for query i iff (not causal or j <= i) and j < L_b,
  where L_b is the key length of batch entry b (N when no lengths are given).
  Masked scores are -inf.  A row with no allowed key has P = 0, O = 0,
  LSE = -inf and zero gradients.
* The saved normaliser is one number per row, LSE_i = m_i + ln(l_i), the natural
  log of the row's softmax denominator in scaled units.
* Dropout: keep mask and scale from oracle.philox (inverted dropout); the row
  normaliser, and hence LSE, is taken before dropout.
* Backward: with Z = keep * s (Z = 1 when p = 0) and P~ = P * Z,
      dV = P~^T dO,  dP = (dO V^T) * Z,  D_i = sum_k dO_ik O_ik,
      dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
  (D_i equals sum_j P_ij dP_ij, the softmax Jacobian contraction.)

Memory: one head's N x N matrices are materialised whole unless `row_chunk` is
given, in which case query rows are evaluated in groups of that many rows.  Each
row's softmax is still computed over its whole row; only the sums over query
rows (dK, dV) are split into partial sums.
"""

import numpy as np

from . import philox


def _as64(x):
    """Widen any float array (fp32, bf16 via torch, fp64) to an fp64 numpy array."""
    if hasattr(x, "detach"):  # a torch tensor: widen on the torch side (bf16 -> f64 is exact)
        import torch

        return x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def allowed_mask(rows, n_keys, causal, key_len):
    """Boolean [len(rows), n_keys]: True where query `rows[r]` may attend key j."""
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(n_keys, dtype=np.int64)[None, :]
    ok = np.broadcast_to(j < int(key_len), (len(rows), n_keys))
    if causal:
        ok = ok & (j <= rows[:, None])
    return ok


def _head_probs(q_rows, k, scale, rows, causal, key_len):
    """Scores, probabilities and LSE for some query rows of one head (fp64)."""
    s = float(scale) * (q_rows @ k.T)
    ok = allowed_mask(rows, k.shape[0], causal, key_len)
    s = np.where(ok, s, -np.inf)
    m = np.max(s, axis=1)
    empty = ~np.isfinite(m)  # rows with no allowed key
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])  # exp(-inf) = 0 for masked entries
    l = np.sum(e, axis=1)
    l_safe = np.where(empty, 1.0, l)
    p = e / l_safe[:, None]
    lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    return p, lse


def _head_z(seed, b, h, rows, n_keys, dropout_p):
    """Dropout multiplier Z = keep * s for the given rows (None when p = 0)."""
    if dropout_p == 0.0:
        return None
    keep = philox.keep_mask(seed, b, h, rows, np.arange(n_keys), dropout_p)
    return keep * philox.dropout_scale(dropout_p)


def _row_groups(n, rows, row_chunk):
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    if row_chunk is None or row_chunk >= len(rows):
        return [rows]
    return [rows[s : s + row_chunk] for s in range(0, len(rows), row_chunk)]


def attention_forward(q, k, v, scale, causal=False, key_lens=None, dropout_p=0.0,
                      seed=0, rows=None, row_chunk=None, heads=None):
    """O and LSE of the attention definition, in fp64.

    q, k, v: [B, H, N, d] (numpy or torch, any float dtype; widened exactly).
    key_lens: None or length-B integers.  rows: optional query rows to evaluate.
    heads: optional list of (b, h) pairs to evaluate (others are left zero).
    Returns (O [B, H, R, d], LSE [B, H, R]) with R = N or len(rows).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, d = q.shape
    nrows = N if rows is None else len(rows)
    out = np.zeros((B, H, nrows, d))
    lse = np.zeros((B, H, nrows))
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in pairs:
        L = N if key_lens is None else int(key_lens[b])
        pos = 0
        for grp in _row_groups(N, rows, row_chunk):
            p, l = _head_probs(q[b, h, grp], k[b, h], scale, grp, causal, L)
            z = _head_z(seed, b, h, grp, N, dropout_p)
            pt = p if z is None else p * z
            out[b, h, pos : pos + len(grp)] = pt @ v[b, h]
            lse[b, h, pos : pos + len(grp)] = l
            pos += len(grp)
    return out, lse


def attention_backward(q, k, v, dout, scale, causal=False, key_lens=None,
                       dropout_p=0.0, seed=0, q_rows=None, k_rows=None,
                       row_chunk=None, heads=None, first_row=0):
    """dQ, dK, dV of the attention definition for upstream gradient dout, in fp64.

    q_rows selects the rows of dQ that are returned, k_rows the rows of dK and
    dV (all by default).  Every query row takes part in dK and dV, so all rows
    are evaluated unless k_rows is empty, in which case only q_rows are.
    heads: optional list of (b, h) pairs to evaluate (others are left zero).
    first_row: with a causal mask, query rows below min(k_rows) never see those
    keys, so only rows >= first_row need evaluating for dK/dV (exact when
    first_row <= min(k_rows); requires causal and explicit k_rows).
    Returns (dQ [B, H, Rq, d], dK [B, H, Rk, d], dV [B, H, Rk, d]).
    """
    q, k, v, dout = _as64(q), _as64(k), _as64(v), _as64(dout)
    B, H, N, d = q.shape
    q_sel = np.arange(N) if q_rows is None else np.asarray(q_rows, dtype=np.int64)
    k_sel = np.arange(N) if k_rows is None else np.asarray(k_rows, dtype=np.int64)
    dq = np.zeros((B, H, len(q_sel), d))
    dk = np.zeros((B, H, len(k_sel), d))
    dv = np.zeros((B, H, len(k_sel), d))
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in pairs:
        L = N if key_lens is None else int(key_lens[b])
        dq_full = np.zeros((N, d)) if q_rows is None else None
        eval_rows = q_sel if len(k_sel) == 0 else None
        if first_row > 0:
            if not causal or k_rows is None or q_rows is None or first_row > int(np.min(k_sel)):
                raise ValueError("first_row needs causal masking, explicit q_rows and k_rows >= first_row")
            eval_rows = np.union1d(np.arange(first_row, N), q_sel)
        for grp in _row_groups(N, eval_rows, row_chunk):
            p, _ = _head_probs(q[b, h, grp], k[b, h], scale, grp, causal, L)
            z = _head_z(seed, b, h, grp, N, dropout_p)
            pt = p if z is None else p * z
            o = pt @ v[b, h]
            do = dout[b, h, grp]
            dv[b, h] += pt[:, k_sel].T @ do
            dp = do @ v[b, h].T
            if z is not None:
                dp = dp * z
            dd = np.sum(do * o, axis=1)
            ds = p * (dp - dd[:, None])
            dk[b, h] += float(scale) * (ds[:, k_sel].T @ q[b, h, grp])
            dq_grp = float(scale) * (ds @ k[b, h])
            if dq_full is not None:
                dq_full[grp] = dq_grp
            else:
                hit = np.isin(q_sel, grp)
                if np.any(hit):
                    pos_in_grp = np.searchsorted(grp, q_sel[hit])
                    dq[b, h, np.nonzero(hit)[0]] = dq_grp[pos_in_grp]
        if dq_full is not None:
            dq[b, h] = dq_full
    return dq, dk, dv


def backward_preprocess(o, dout):
    """D_i = sum_k dO_ik O_ik per row (fp64), shape [B, H, N]."""
    return np.sum(_as64(o) * _as64(dout), axis=-1)
