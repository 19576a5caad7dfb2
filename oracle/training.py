"""fp64 oracle of one synthetic training step with a banded Sinkhorn attention layer.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the product path.

The pages validate trainability on a masked protein-embedding reconstruction task: embeddings
go through the Sinkhorn attention layer, a reconstruction loss is taken, the exact tail VJP
carries its gradient back, and an optimiser updates the weights (technical summaries §4.2 and
atlas, Experimental setup: reconstruction MSE on Pfam ESM-2 embeddings).  The data are not
available, and the pages fix neither the model around the layer nor the optimiser; the plainest
model that has every named part is read here (listed in the design notes):

  X [B, L, D] embeddings; mask [B, L] in {0, 1} marks the tokens to reconstruct;
  Xin = X with masked tokens zeroed;
  Q = Xin Wq, K = Xin Wk, V = Xin Wv, split into H = D / d heads of width d;
  O_h = banded balanced Sinkhorn attention of (Q_h, K_h, V_h) (stopped T-step base, R-step
        tail; the forward and one-reference VJP of sinkhorn_band), heads merged back to [B, L, D];
  Y = O Wo;
  loss = sum over masked tokens of ||Y_t - X_t||^2 / (number of masked tokens * D);
  plain SGD: W <- W - lr dloss/dW for W in (Wq, Wk, Wv, Wo).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .sinkhorn_band import BandProblem, forward, vjp_one_reference, vjp_tail_one_reference


@dataclass(frozen=True)
class TrainConfig:
    heads: int
    W: int
    T: int
    R: int
    eps: float = 1.0
    lr: float = 0.1


def _split(X, H):
    """[B, L, D] -> [B, H, L, D / H]"""
    B, L, D = X.shape
    return X.reshape(B, L, H, D // H).transpose(0, 2, 1, 3)


def _merge(Xh):
    """[B, H, L, d] -> [B, L, H d]"""
    B, H, L, d = Xh.shape
    return Xh.transpose(0, 2, 1, 3).reshape(B, L, H * d)


def reconstruction_step(params, X, mask, cfg: TrainConfig, want_duals: bool = False):
    """One step of the masked-reconstruction model: (loss, grads, new_params), each of grads and
    new_params a tuple (Wq, Wk, Wv, Wo) of [D, D] arrays (and the per-head saved duals if
    want_duals).
    [technical summaries §4.2: the layer trained end to end on a reconstruction objective;
    §2.1-§2.2: the attention forward and its exact tail VJP]"""
    Wq, Wk, Wv, Wo = (np.asarray(w, dtype=np.float64) for w in params)
    X = np.asarray(X, dtype=np.float64)
    mask = np.asarray(mask, dtype=np.float64)
    B, L, D = X.shape
    H = cfg.heads
    prob = BandProblem(W=cfg.W, T=cfg.T, R=cfg.R, eps=cfg.eps)
    vjp = vjp_one_reference if cfg.R == 2 else vjp_tail_one_reference

    Xin = X * (1.0 - mask)[..., None]
    Q, K, V = Xin @ Wq, Xin @ Wk, Xin @ Wv
    Qh, Kh, Vh = _split(Q, H), _split(K, H), _split(V, H)
    Oh = np.zeros_like(Qh)
    duals = {}
    for b in range(B):
        for h in range(H):
            Oh[b, h], duals[b, h] = forward(Qh[b, h], Kh[b, h], Vh[b, h], prob)
    O = _merge(Oh)
    Y = O @ Wo
    n = float(mask.sum()) * D
    diff = (Y - X) * mask[..., None]
    loss = float(np.sum(diff ** 2) / n)

    dY = 2.0 * diff / n
    dWo = O.reshape(-1, D).T @ dY.reshape(-1, D)
    dOh = _split(dY @ Wo.T, H)
    dQh, dKh, dVh = np.zeros_like(Qh), np.zeros_like(Qh), np.zeros_like(Qh)
    for b in range(B):
        for h in range(H):
            dQh[b, h], dKh[b, h], dVh[b, h] = vjp(Qh[b, h], Kh[b, h], Vh[b, h], dOh[b, h],
                                                  duals[b, h], prob)
    Xf = Xin.reshape(-1, D)
    dWq = Xf.T @ _merge(dQh).reshape(-1, D)
    dWk = Xf.T @ _merge(dKh).reshape(-1, D)
    dWv = Xf.T @ _merge(dVh).reshape(-1, D)
    grads = (dWq, dWk, dWv, dWo)
    new = tuple(w - cfg.lr * g for w, g in zip((Wq, Wk, Wv, Wo), grads))
    if want_duals:
        return loss, grads, new, duals
    return loss, grads, new


def reconstruction_loss(params, X, mask, cfg: TrainConfig, base=None) -> float:
    """The loss alone (the forward half of reconstruction_step).  With base = the per-head saved
    duals of an earlier forward ({(b, h): duals}), each head's stopped base state is held at
    those values instead of being re-solved: this is the function the step's gradient
    differentiates (stop-gradient on the base)."""
    from .sinkhorn_band import forward_from_base
    Wq, Wk, Wv, Wo = (np.asarray(w, dtype=np.float64) for w in params)
    X = np.asarray(X, dtype=np.float64)
    mask = np.asarray(mask, dtype=np.float64)
    B, L, D = X.shape
    H = cfg.heads
    prob = BandProblem(W=cfg.W, T=cfg.T, R=cfg.R, eps=cfg.eps)
    Xin = X * (1.0 - mask)[..., None]
    Qh, Kh, Vh = _split(Xin @ Wq, H), _split(Xin @ Wk, H), _split(Xin @ Wv, H)
    Oh = np.zeros_like(Qh)
    for b in range(B):
        for h in range(H):
            if base is None:
                Oh[b, h] = forward(Qh[b, h], Kh[b, h], Vh[b, h], prob)[0]
            else:
                d0 = base[b, h]
                u0 = d0[0] if cfg.R == 0 else None
                Oh[b, h] = forward_from_base(Qh[b, h], Kh[b, h], Vh[b, h], d0[-1] if cfg.R == 0
                                             else d0[0], prob, u0=u0)
    diff = (_merge(Oh) @ Wo - X) * mask[..., None]
    return float(np.sum(diff ** 2) / (float(mask.sum()) * D))
