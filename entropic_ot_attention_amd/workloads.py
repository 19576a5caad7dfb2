"""Seeded synthetic workloads for banded balanced Sinkhorn attention.

This module only names problem shapes and draws seeded random inputs; it holds
none of the method's arithmetic, so both the HIP path's tests and the fp64 CPU
checker can take their inputs from it.

Inputs are i.i.d. N(0, 1) float32 drawn from ``torch.Generator('cpu')`` seeded per
workload, in the order Q, K, V, dO, each shaped [batch, heads, L, d] and viewed as
[batch*heads, L, d].  bf16 workloads round those draws to bfloat16 (round to
nearest even) before either side sees them.  The pages train on Pfam ESM-2
embeddings, which are not available here; Gaussian embeddings of the same head
dimension stand in for them.
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    L: int            # tokens per sequence (dustbin workloads: real tokens, the dustbin is extra)
    d: int
    W: int            # band width, support |i - j| <= W // 2
    T: int            # stopped base steps
    R: int            # tail steps
    eps: float
    dtype: str        # "f32" or "bf16"
    seed: int
    dustbin: bool = False

    @property
    def bh(self) -> int:
        return self.batch * self.heads

    @property
    def tokens(self) -> int:
        """Token rows held per (batch, head) problem (dustbin workloads add one)."""
        return self.L + (1 if self.dustbin else 0)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five named workloads.  Names state what they are.
TINY_L512 = Workload("tiny_L512_W64_f32", 1, 1, 512, 64, 64, 15, 2, 1.0, "f32", 0)
BATCH_L2048 = Workload("batch4x8_L2048_W128_f32", 4, 8, 2048, 64, 128, 15, 2, 1.0, "f32", 1)
HEADS8_L32K = Workload("heads8_L32768_W256_T20_bf16", 1, 8, 32768, 64, 256, 20, 2, 1.0, "bf16", 2)
LONG_L262K = Workload("seq1x4_L262144_W256_bf16", 1, 4, 262144, 64, 256, 15, 2, 1.0, "bf16", 3)
DUSTBIN_L4096 = Workload("dustbin_block_L4096p1_f32", 1, 4, 4096, 64, 256, 15, 2, 1.0, "f32", 4,
                         dustbin=True)

WORKLOADS = {w.name: w for w in (TINY_L512, BATCH_L2048, HEADS8_L32K, LONG_L262K, DUSTBIN_L4096)}


def make_inputs(w: Workload, with_cotangent: bool = True):
    """Seeded Q, K, V (and dO) of shape [bh, tokens, d] in the workload's dtype (CPU)."""
    g = torch.Generator("cpu").manual_seed(w.seed)
    shape = (w.batch, w.heads, w.tokens, w.d)
    names = ("Q", "K", "V", "dO") if with_cotangent else ("Q", "K", "V")
    out = {}
    for n in names:
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        out[n] = x.reshape(w.bh, w.tokens, w.d).to(w.torch_dtype).contiguous()
    return out


@dataclass(frozen=True)
class TrainWorkload:
    """Masked-reconstruction training step: batch x L tokens of D-wide embeddings (D = 64 heads),
    a fraction `masked` of the tokens to reconstruct, band W, T base and R tail steps."""
    name: str
    batch: int
    L: int
    D: int
    W: int
    T: int
    R: int
    eps: float
    masked: float
    lr: float
    compute: str      # "f32" or "bf16"
    seed: int

    @property
    def heads(self) -> int:
        return self.D // 64

    @property
    def torch_dtype(self):
        return torch.float32 if self.compute == "f32" else torch.bfloat16

    def with_(self, **kw) -> "TrainWorkload":
        return replace(self, **kw)


# One device's share of the pages' data-parallel run (64 examples per step over 8 devices) at
# the width of ESM-2 650M embeddings (1280 = 20 heads of 64) and Pfam-domain lengths.
TRAIN_B8_L1024 = TrainWorkload("train_b8_L1024_D1280_W256_T15_bf16", 8, 1024, 1280, 256, 15, 2,
                               1.0, 0.15, 0.05, "bf16", 5)

TRAIN_WORKLOADS = {w.name: w for w in (TRAIN_B8_L1024,)}


# Correlation of neighbouring tokens' embeddings in the synthetic training sequences
TRAIN_RHO = 0.9


def make_training_batch(w: TrainWorkload):
    """Seeded embeddings X [batch, L, D], mask [batch, L] (Bernoulli(masked), at least one masked
    token per example) and weights (Wq, Wk, Wv, Wo) ~ N(0, 1 / D), fp32 on the CPU, drawn in that
    order.  The embeddings are a stationary AR(1) sequence along the tokens,
    X_t = rho X_(t-1) + sqrt(1 - rho^2) e_t with e ~ N(0, 1) and rho = TRAIN_RHO, so that, as in
    real sequences, a masked token is predictable from its neighbours in the band."""
    g = torch.Generator("cpu").manual_seed(w.seed)
    E = torch.randn((w.batch, w.L, w.D), generator=g, dtype=torch.float32)
    X = torch.empty_like(E)
    X[:, 0] = E[:, 0]
    c = (1.0 - TRAIN_RHO ** 2) ** 0.5
    for t in range(1, w.L):
        X[:, t] = TRAIN_RHO * X[:, t - 1] + c * E[:, t]
    mask = (torch.rand((w.batch, w.L), generator=g) < w.masked).to(torch.float32)
    mask[:, 0] = 1.0
    weights = tuple(torch.randn((w.D, w.D), generator=g, dtype=torch.float32) / w.D ** 0.5
                    for _ in range(4))
    return X, mask, weights
