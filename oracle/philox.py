"""Philox4x32-10 counter-based generator and the dropout keep mask built on it.

TEST INFRASTRUCTURE ONLY.  This package is the CPU oracle that the GPU path is
checked against.  Only the test suite, the smoke check and the CPU-baseline leg
of the benchmark may import it; the library and its Python binding never do.

What the pages fix: dropout is applied element-wise to the attention
probabilities after the softmax and before the product with V (FlashAttention
first principles, section 2 and section 4.1 "why attention is slow").  They do not say
which generator draws the mask.  The reading used here (stated once, used by
both sides): a Philox4x32-10 generator keyed by the 64-bit seed, whose counter
is built from (batch b, head h, query row i, key column j).

Philox4x32-10 is the generator of Salmon, Moraes, Dror and Shaw, "Parallel
Random Numbers: As Easy as 1, 2, 3" (SC'11).  One round maps a 4-word counter
(c0, c1, c2, c3) under a 2-word key (k0, k1) to

    (hi(B*c2) ^ c1 ^ k0,  lo(B*c2),  hi(A*c0) ^ c3 ^ k1,  lo(A*c0))

where A = 0xD2511F53, B = 0xCD9E8D57 and hi/lo are the halves of the 64-bit
product.  Ten rounds are applied; between consecutive rounds the key is bumped
by the Weyl constants (0x9E3779B9, 0xBB67AE85), all arithmetic modulo 2**32.

Counter and key layout for the dropout mask of element (b, h, i, j):
    key     = (low 32 bits of seed, high 32 bits of seed)
    counter = (j >> 2, i, h, b)
    word    = output word number (j & 3)
so one generator call serves four neighbouring key columns of one query row.
Keep the element iff word >= T with T = floor(p * 2**32), p taken as the fp32
value passed to the library and widened to fp64.  Kept elements are scaled by
s = fp32(1 / (1 - p)) (inverted dropout), again computed in fp64 and rounded
once to fp32.
"""

import numpy as np

PHILOX_M0 = 0xD2511F53  # multiplier applied to counter word 0
PHILOX_M1 = 0xCD9E8D57  # multiplier applied to counter word 2
PHILOX_W0 = 0x9E3779B9  # key bump for key word 0
PHILOX_W1 = 0xBB67AE85  # key bump for key word 1
MASK32 = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """Apply Philox4x32-10 to counters.

    counter: integer array [..., 4] (values < 2**32), key: integer array [..., 2]
    broadcastable against counter[..., :2].  Returns uint32 array [..., 4].
    Arithmetic is carried in uint64 so the 32x32->64 products are exact.
    """
    c = np.asarray(counter, dtype=np.uint64)
    k = np.asarray(key, dtype=np.uint64)
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0 = np.broadcast_to(k[..., 0], c0.shape).copy()
    k1 = np.broadcast_to(k[..., 1], c0.shape).copy()
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    w0 = np.uint64(PHILOX_W0)
    w1 = np.uint64(PHILOX_W1)
    mask = np.uint64(MASK32)
    shift = np.uint64(32)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + w0) & mask
            k1 = (k1 + w1) & mask
        p0 = m0 * c0  # < 2**64, exact in uint64
        p1 = m1 * c2
        hi0, lo0 = p0 >> shift, p0 & mask
        hi1, lo1 = p1 >> shift, p1 & mask
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def seed_key(seed):
    """The generator key: (low word, high word) of the 64-bit seed."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return np.array([seed & MASK32, seed >> 32], dtype=np.uint64)


def dropout_threshold(p):
    """T = floor(p * 2**32) with p the fp32 dropout probability widened to fp64."""
    p64 = float(np.float32(p))
    if not (0.0 <= p64 < 1.0):
        raise ValueError("dropout probability must lie in [0, 1)")
    return int(np.floor(p64 * 4294967296.0))


def dropout_scale(p):
    """s = fp32(1 / (1 - p)), returned as the exact fp32 value in a Python float."""
    p64 = float(np.float32(p))
    return float(np.float32(1.0 / (1.0 - p64)))


def keep_mask(seed, b, h, rows, cols, p):
    """Boolean keep mask for query rows `rows` x key columns `cols` of head (b, h).

    rows, cols: 1-D integer arrays.  Element (i, j) is kept iff the Philox word
    number (j & 3) of counter (j >> 2, i, h, b) is >= floor(p * 2**32).
    """
    rows = np.asarray(rows, dtype=np.uint64)
    cols = np.asarray(cols, dtype=np.uint64)
    ii, jj = np.meshgrid(rows, cols, indexing="ij")
    counter = np.stack(
        [jj >> np.uint64(2), ii, np.full_like(ii, h), np.full_like(ii, b)], axis=-1
    )
    words = philox4x32_10(counter, seed_key(seed))
    pick = (jj & np.uint64(3)).astype(np.int64)
    r = np.take_along_axis(words, pick[..., None], axis=-1)[..., 0]
    return r.astype(np.uint64) >= np.uint64(dropout_threshold(p))
