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
