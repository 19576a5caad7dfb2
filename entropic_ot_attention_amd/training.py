"""Synthetic training step around the banded Sinkhorn attention layer.

The pages train the layer end to end on masked protein-embedding reconstruction (technical
summaries §4.2; atlas, Experimental setup).  This module is that step on seeded synthetic
embeddings: masked tokens zeroed in the input, Q/K/V projections, multi-head banded balanced
Sinkhorn attention through the HIP library (SinkhornAttention: forward and exact tail VJP), an
output projection, mean squared error over the masked tokens, and a plain SGD update.  The
projections, loss and update are torch library operations (rocBLAS / hipBLASLt GEMMs and
elementwise kernels); every step of the attention runs in the library.

compute_dtype bfloat16 runs the projections and the attention on bf16 copies of the inputs and
weights (fp32 accumulation in the GEMMs and in the attention, fp32 duals), with fp32 master
weights, loss and update.
"""

from __future__ import annotations

import torch

from .autograd import sinkhorn_attention


class ReconstructionModel(torch.nn.Module):
    def __init__(self, weights, heads: int, W: int, T: int, R: int = 2, epsilon: float = 1.0,
                 compute_dtype: torch.dtype = torch.float32, schedule: str = "one_reference"):
        super().__init__()
        Wq, Wk, Wv, Wo = weights
        D = Wq.shape[0]
        if D % heads != 0 or D // heads != 64:
            raise ValueError("the attention runs heads of width 64: D must be 64 * heads")
        self.Wq = torch.nn.Parameter(Wq.clone())
        self.Wk = torch.nn.Parameter(Wk.clone())
        self.Wv = torch.nn.Parameter(Wv.clone())
        self.Wo = torch.nn.Parameter(Wo.clone())
        self.heads, self.W, self.T, self.R, self.eps = heads, W, T, R, epsilon
        self.compute_dtype = compute_dtype
        self.schedule = schedule

    @property
    def weights(self):
        return (self.Wq, self.Wk, self.Wv, self.Wo)

    def forward(self, X, mask):
        """Mean squared reconstruction error over the masked tokens; X [B, L, D] fp32,
        mask [B, L] (1 = reconstruct)."""
        B_, L, D = X.shape
        H, d = self.heads, D // self.heads
        cd = self.compute_dtype
        Xin = (X * (1.0 - mask)[..., None]).to(cd)

        def heads_of(Z):
            return Z.view(B_, L, H, d).permute(0, 2, 1, 3).contiguous().view(B_ * H, L, d)

        Q = heads_of(Xin @ self.Wq.to(cd))
        K = heads_of(Xin @ self.Wk.to(cd))
        V = heads_of(Xin @ self.Wv.to(cd))
        O = sinkhorn_attention(Q, K, V, self.W, self.T, self.R, self.eps, self.schedule)
        O = O.view(B_, H, L, d).permute(0, 2, 1, 3).contiguous().view(B_, L, D)
        Y = (O @ self.Wo.to(cd)).float()
        diff = (Y - X) * mask[..., None]
        return (diff * diff).sum() / (mask.sum() * D)


def sgd_step(model: ReconstructionModel, X, mask, lr: float):
    """One training step: loss, weight gradients (fp32), and W <- W - lr grad in place."""
    loss = model(X, mask)
    grads = torch.autograd.grad(loss, model.weights)
    with torch.no_grad():
        for w, g in zip(model.weights, grads):
            w.sub_(lr * g.float())
    return loss.detach(), grads
