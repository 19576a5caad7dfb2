"""Implementations that share no code with the oracle, used only to pin it.

* ``textbook_sinkhorn``: multiplicative Sinkhorn-Knopp matrix scaling on a dense
  matrix (a = 1 / (A b), b = 1 / (A^T a)), no log domain, no band storage.
* ``dense_autograd``: the stopped-base tail surrogate written with dense [L, L]
  torch float64 tensors and differentiated by torch autograd on the CPU
  ("exact autodiff through the surrogate", the pages' validation baseline).
* ``dense_autograd_full``: the same iteration with gradients flowing through the base steps
  as well (full backpropagation through time).
* ``cross_ratio_diameter``: the projective diameter of a positive matrix by enumerating every
  2 x 2 minor's log cross ratio of the exponentiated matrix (Birkhoff's definition).
* ``dense_reconstruction_grads``: the masked-reconstruction model around the attention layer in
  dense torch float64, its stopped-base surrogate differentiated by torch autograd.
"""

from __future__ import annotations

import math

import numpy as np
import torch


def dense_scores(Q, K, W, eps):
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    L, d = Q.shape
    S = Q @ K.T / (math.sqrt(d) * eps)
    i = np.arange(L)
    mask = np.abs(i[:, None] - i[None, :]) <= W // 2
    return S, mask


def textbook_sinkhorn(A: np.ndarray, steps: int):
    """Sinkhorn-Knopp scaling of a nonnegative matrix to unit row and column sums.
    Starts from b = 1; each step sets a = 1/(A b) then b = 1/(A^T a).
    Returns (a, b) after `steps` steps (a = None when steps == 0)."""
    b = np.ones(A.shape[1])
    a = None
    for _ in range(steps):
        a = 1.0 / (A @ b)
        b = 1.0 / (A.T @ a)
    return a, b


def dense_autograd(Q, K, V, dO, W, T, R, eps):
    """Dense-matrix surrogate: stopped T-step base, R-step tail, O = P^(R,R) V.
    Returns (O, dQ, dK, dV, duals) with duals = [v0, u1, v1, ..., uR, vR] ([u0, v0] for
    R = 0, when the output plan is the stopped base's own)."""
    Qt = torch.tensor(np.asarray(Q, np.float64), requires_grad=True)
    Kt = torch.tensor(np.asarray(K, np.float64), requires_grad=True)
    Vt = torch.tensor(np.asarray(V, np.float64), requires_grad=True)
    dOt = torch.tensor(np.asarray(dO, np.float64))
    L, d = Qt.shape
    idx = torch.arange(L)
    mask = (idx[:, None] - idx[None, :]).abs() <= W // 2
    S = (Qt @ Kt.T) / (math.sqrt(d) * eps)
    S = S.masked_fill(~mask, float("-inf"))
    with torch.no_grad():
        u = torch.zeros(L, dtype=torch.float64)
        v = torch.zeros(L, dtype=torch.float64)
        Sd = S.detach()
        for _ in range(T):
            u = -torch.logsumexp(Sd + v[None, :], dim=1)
            v = -torch.logsumexp(Sd + u[:, None], dim=0)
    v = v.detach()
    duals = [u.detach(), v] if R == 0 else [v]
    for _ in range(R):
        u = -torch.logsumexp(S + v[None, :], dim=1)
        v = -torch.logsumexp(S + u[:, None], dim=0)
        duals += [u, v]
    P = torch.exp(S + u[:, None] + v[None, :])
    O = P @ Vt
    (O * dOt).sum().backward()
    return (O.detach().numpy(), Qt.grad.numpy(), Kt.grad.numpy(), Vt.grad.numpy(),
            np.stack([x.detach().numpy() for x in duals]))


def dense_autograd_full(Q, K, V, dO, W, T, R, eps):
    """Dense-matrix iteration with no stop-gradient: T base steps and R tail steps, all
    differentiated.  Returns (O, dQ, dK, dV)."""
    Qt = torch.tensor(np.asarray(Q, np.float64), requires_grad=True)
    Kt = torch.tensor(np.asarray(K, np.float64), requires_grad=True)
    Vt = torch.tensor(np.asarray(V, np.float64), requires_grad=True)
    dOt = torch.tensor(np.asarray(dO, np.float64))
    L, d = Qt.shape
    idx = torch.arange(L)
    mask = (idx[:, None] - idx[None, :]).abs() <= W // 2
    S = (Qt @ Kt.T) / (math.sqrt(d) * eps)
    S = S.masked_fill(~mask, float("-inf"))
    u = torch.zeros(L, dtype=torch.float64)
    v = torch.zeros(L, dtype=torch.float64)
    for _ in range(T + R):
        u = -torch.logsumexp(S + v[None, :], dim=1)
        v = -torch.logsumexp(S + u[:, None], dim=0)
    P = torch.exp(S + u[:, None] + v[None, :])
    O = P @ Vt
    (O * dOt).sum().backward()
    return O.detach().numpy(), Qt.grad.numpy(), Kt.grad.numpy(), Vt.grad.numpy()


def cross_ratio_diameter(A):
    """max over i, i', j, j' of log(A_ij A_i'j' / (A_ij' A_i'j)) for a strictly positive A,
    every quadruple enumerated."""
    A = np.asarray(A, dtype=np.float64)
    n, m = A.shape
    best = 0.0
    for i in range(n):
        for i2 in range(n):
            for j in range(m):
                for j2 in range(m):
                    best = max(best, math.log((A[i, j] * A[i2, j2]) / (A[i, j2] * A[i2, j])))
    return best


def _dense_surrogate_heads(Q, K, V, W, T, R, eps):
    """Stopped-base tail surrogate for [n, L, d] tensors in the autograd graph: O = P^(R,R) V."""
    n, L, d = Q.shape
    idx = torch.arange(L)
    band = (idx[:, None] - idx[None, :]).abs() <= W // 2
    S = (Q @ K.transpose(1, 2)) / (math.sqrt(d) * eps)
    S = S.masked_fill(~band, float("-inf"))
    with torch.no_grad():
        u = torch.zeros(n, L, dtype=S.dtype)
        v = torch.zeros(n, L, dtype=S.dtype)
        for _ in range(T):
            u = -torch.logsumexp(S + v[:, None, :], dim=2)
            v = -torch.logsumexp(S + u[:, :, None], dim=1)
    u, v = u.detach(), v.detach()
    for _ in range(R):
        u = -torch.logsumexp(S + v[:, None, :], dim=2)
        v = -torch.logsumexp(S + u[:, :, None], dim=1)
    P = torch.exp(S + u[:, :, None] + v[:, None, :])
    return P @ V


def dense_reconstruction_grads(params, X, mask, heads, W, T, R, eps):
    """(loss, (dWq, dWk, dWv, dWo)) of the masked-reconstruction model: masked tokens zeroed in
    the input, Q/K/V projections, per-head stopped-base Sinkhorn attention, output projection,
    mean squared error over the masked tokens' D features; torch float64 autograd."""
    Ws = [torch.tensor(np.asarray(w, np.float64), requires_grad=True) for w in params]
    Xt = torch.tensor(np.asarray(X, np.float64))
    m = torch.tensor(np.asarray(mask, np.float64))
    B, L, D = Xt.shape
    d = D // heads
    Xin = Xt * (1 - m)[..., None]

    def heads_of(Z):
        return Z.reshape(B, L, heads, d).permute(0, 2, 1, 3).reshape(B * heads, L, d)

    Q, K, V = (heads_of(Xin @ Ws[k]) for k in range(3))
    O = _dense_surrogate_heads(Q, K, V, W, T, R, eps)
    O = O.reshape(B, heads, L, d).permute(0, 2, 1, 3).reshape(B, L, D)
    Y = O @ Ws[3]
    loss = (((Y - Xt) * m[..., None]) ** 2).sum() / (m.sum() * D)
    loss.backward()
    return float(loss.detach()), tuple(w.grad.numpy() for w in Ws)
