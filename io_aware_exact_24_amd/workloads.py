"""Seeded synthetic inputs for the attention workloads.

This module draws inputs only; it holds none of the attention arithmetic and
imports nothing from the library or the oracle, so both sides can be fed the
same bits from it.

The pages measure on model training runs (BERT-large at 512 tokens, GPT-2 at
1024, ViT-Huge at 2048, long protein sequences; Flash Attention hardware-aware
optimisation, section 3.1) that need datasets and trained weights.  Standing in for
them: i.i.d. N(0, 1) tensors of the attention shapes below, drawn in fp32 on the
CPU from torch.Generator().manual_seed(1000 + config number) in the order Q, K,
V, dO, then rounded to the workload dtype (round-to-nearest-even).  With scale
1/sqrt(d) the scores then have about unit variance.
"""

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

DROPOUT_SEED = 0x0123456789ABCDEF  # Philox key used by the dropout workload


@dataclass(frozen=True)
class Workload:
    number: int
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "f32" or "bf16"
    causal: bool = False
    padded: bool = False  # key lengths drawn uniformly from [N/4, N]
    dropout_p: float = 0.0
    backward: bool = True
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        """fp32(1/sqrt(d)) as a Python float (the exact value handed to the library)."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def seed(self) -> int:
        return 1000 + self.number

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    1: Workload(1, "single_head_fp32", 1, 1, 128, 64, "f32", backward=False,
                note="single head, forward only, fp32"),
    2: Workload(2, "bert_large_like", 8, 16, 1024, 64, "bf16",
                note="multi-head, non-causal"),
    3: Workload(3, "decoder_causal", 4, 32, 4096, 128, "bf16", causal=True,
                note="causal decoder shape"),
    4: Workload(4, "padded_dropout", 16, 12, 2048, 64, "bf16", padded=True, dropout_p=0.1,
                note="key padding + Philox dropout p=0.1"),
    5: Workload(5, "long_causal", 1, 8, 65536, 64, "bf16", causal=True,
                note="long sequence, causal"),
}


@dataclass
class Inputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    dout: torch.Tensor
    key_lens: Optional[torch.Tensor]  # int32 [B] on the CPU, or None


def draw(B, H, N, d, dtype=torch.bfloat16, seed=0, padded=False, dout=True,
         q_mult=1.0):
    """Draw Q, K, V (and dO) as N(0,1) fp32, rounded to `dtype`, on the CPU.

    q_mult scales Q before rounding (a peaked-softmax variant).  When `padded`,
    key lengths are then drawn uniformly from [N // 4, N].
    """
    g = torch.Generator().manual_seed(seed)
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    if q_mult != 1.0:
        q = q * q_mult
    q = q.to(dtype)
    k = torch.randn(shape, generator=g, dtype=torch.float32).to(dtype)
    v = torch.randn(shape, generator=g, dtype=torch.float32).to(dtype)
    do = torch.randn(shape, generator=g, dtype=torch.float32).to(dtype) if dout else None
    key_lens = None
    if padded:
        key_lens = torch.randint(N // 4, N + 1, (B,), generator=g, dtype=torch.int32)
    return Inputs(q, k, v, do, key_lens)


def draw_workload(w: Workload):
    return draw(w.B, w.H, w.N, w.d, w.torch_dtype, w.seed, padded=w.padded)


def sampled_rows(N, seed, count=64):
    """Rows checked at sizes the oracle cannot evaluate whole.

    Tile and tail edges plus random rows drawn from `seed`; sorted, unique,
    at most max(count, number of edge rows) of them.
    """
    fixed = sorted({r for r in (0, 1, 63, 64, 127, 128, N // 2, N - 2, N - 1) if 0 <= r < N})
    rng = np.random.default_rng(seed)
    pool = np.setdiff1d(np.arange(N), fixed)
    extra = rng.choice(pool, size=min(len(pool), max(0, count - len(fixed))), replace=False)
    return np.unique(np.concatenate([np.array(fixed, dtype=np.int64), extra.astype(np.int64)]))
