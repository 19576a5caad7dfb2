"""fp64 oracle of the projective contraction certificate of the Sinkhorn map's active blocks.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the product path.

Method (technical summaries, gist.science de/fr, §2.4, the projective contraction
certificate; atlas.scime.ai, "Builds on": Birkhoff-Hopf contraction): Hilbert's projective
metric shows that a strictly positive block of the Sinkhorn map is a contraction.  For a
strictly positive matrix A the Birkhoff-Hopf theorem bounds the contraction of x -> A x in
that metric by kappa(A) = tanh(Delta(A) / 4), where the projective diameter is the largest
log cross ratio

    Delta(A) = max over rows i, i' and columns j, j' of  log(A_ij A_i'j' / (A_ij' A_i'j)).

With the Gibbs kernel A = exp(S) of the attention scores the cross ratio is a sum of scores,
so Delta = max over row pairs (i, i') of the oscillation max_j - min_j of S_ij - S_i'j.  In
the log domain a row half-step u = -log(A e^v) then satisfies
osc(u(v1) - u(v2)) <= kappa(A) osc(v1 - v2) (the reciprocal is a Hilbert isometry), and a
full (row, column) step contracts by kappa(A) kappa(A^T) = kappa(A)^2.

Reading where the pages are silent (listed in the design notes): the active blocks are the
tiles of a partition of the token axis into blocks of B tokens (the last one ragged); a block
pair (row block rb, column block cb) is active when every pair in it lies on the support, so
its kernel block is strictly positive.  Blocks reaching off the support have zero entries,
where the diameter is infinite and no contraction is certified; they are reported as -1.
For the dustbin_block support (every pair of the L + 1 active tokens) every block is active.
"""

from __future__ import annotations

import numpy as np

from .sinkhorn_band import BandProblem


def block_layout(n_tokens: int, h: int, block: int):
    """(nb, m): nb = ceil(n_tokens / B) row (and column) blocks; a block pair at column-block
    offset o = cb - rb can be active only if |o| B <= h, so offsets run over -m..m with
    m = min(h // B, nb - 1)."""
    nb = -(-n_tokens // block)
    m = min(h // block, max(nb - 1, 0))
    return nb, m


def block_diameters(Q, K, prob: BandProblem, block: int = 16, dustbin: bool = False):
    """Projective diameter Delta of every active B x B block of the kernel exp(S), S = q.k /
    (sqrt(d) eps), laid out as [nb, 2 m + 1] by (row block, offset + m); -1 where the block
    pair is not active or does not exist.  dustbin=True takes the dustbin_block support: Q, K
    hold the L + 1 active tokens (the dustbin last) and every pair of them is on the support.
    [technical summaries §2.4: projective contraction certificate of strictly positive active
    blocks; §2.3: the dustbin augmentation's dense active support]"""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    n, d = Q.shape
    h = max(prob.h, n - 1) if dustbin else prob.h
    nb, m = block_layout(n, h, block)
    delta = np.full((nb, 2 * m + 1), -1.0)
    scale = 1.0 / (np.sqrt(d) * prob.eps)
    for rb in range(nb):
        r0, r1 = rb * block, min(rb * block + block, n)
        for o in range(-m, m + 1):
            cb = rb + o
            if cb < 0 or cb >= nb:
                continue
            c0, c1 = cb * block, min(cb * block + block, n)
            if max(r1 - 1 - c0, c1 - 1 - r0) > h:
                continue                      # some pair off the support: not strictly positive
            S = (Q[r0:r1] @ K[c0:c1].T) * scale
            diff = S[:, None, :] - S[None, :, :]          # [i, i', j] = S_ij - S_i'j
            delta[rb, o + m] = float(np.max(diff.max(axis=2) - diff.min(axis=2)))
    return delta


def contraction_coefficients(delta):
    """Birkhoff-Hopf coefficient kappa = tanh(Delta / 4) of each active block (-1 elsewhere).
    [technical summaries §2.4; atlas "Builds on": Birkhoff-Hopf contraction]"""
    delta = np.asarray(delta, dtype=np.float64)
    return np.where(delta >= 0, np.tanh(np.maximum(delta, 0.0) / 4.0), -1.0)
