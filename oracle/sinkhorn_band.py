"""fp64 band-storage oracle: banded balanced Sinkhorn attention, forward and R-step tail VJP.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the product path.

Storage.  One head at a time.  Scores and plans live on the fixed band support
Omega = {(i, j): |i - j| <= h}, h = W // 2, stored by diagonal: ``X[k, i]`` is the
entry (i, j = i + k - h).  Entries off Omega (j < 0, j >= L, or an inactive token)
hold -inf for scores and 0 for plans.  Column-indexed views ``Xc[k, j]`` hold the
same entry (i = j - (k - h), j) and are produced by shifting each diagonal.

Method, as stated on the pages (technical summaries, gist.science de/fr, §2.1-§2.3;
abstract):
  * the support is a fixed band of width W, the entropic temperature is absorbed
    into the scores: S_ij = q_i . k_j / (sqrt(d) * epsilon) on Omega;
  * a stopped T-step balanced Sinkhorn solve gives the base duals;
  * a short differentiable tail of R steps refines them, starting from the
    stopped base; the tail is differentiated exactly;
  * for R = 2 the adjoint involves the staircase plans P^(2,2), P^(2,1), P^(1,1),
    P^(1,0), all in one row/column scaling orbit of P^(2,2)
    (orbit equation in §2.2): P^(a,b) = P^(2,2) * exp(u^(a) - u^(2)) * exp(v^(b) - v^(2)).

Readings where the pages are silent (each is listed with its justification in
the design notes of this repository):
  * support |i - j| <= W/2;  balanced = unit row and unit column marginals;
  * cold start u = v = 0; each Sinkhorn step is a row (u) update followed by a
    column (v) update, which is the order the staircase names P^(1,0), P^(1,1),
    P^(2,1), P^(2,2) imply (u^(1) is formed against v^(0));
  * T and R count full (u, v) steps; the base stops after exactly T steps and
    only v^(0) is read by the tail (stop-gradient on the whole base);
  * the output is O = P^(R,R) V (the reference plan, columns exactly balanced);
  * the "centered" surrogate differs from this one by a gauge shift of the stopped
    duals, which changes no plan (tested as an invariant, not applied).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

NEG_INF = -np.inf


@dataclass(frozen=True)
class BandProblem:
    """Problem constants: band width W (support |i-j| <= W//2), T base steps,
    R tail steps, temperature epsilon (scores are q.k / (sqrt(d) * epsilon)).
    R = 0 (no differentiable tail) takes the plan of the stopped base itself, whose duals
    (u^(0), v^(0)) the base must have produced: it needs T >= 1."""

    W: int
    T: int
    R: int
    eps: float = 1.0

    def __post_init__(self):
        if self.R < 0 or self.T < 0:
            raise ValueError("T and R must be >= 0")
        if self.R == 0 and self.T == 0:
            raise ValueError("R = 0 needs T >= 1: the plan's duals come from the base")

    @property
    def h(self) -> int:
        return self.W // 2


# --------------------------------------------------------------------------------------
# band bookkeeping (pure index manipulation, no arithmetic of the method)
# --------------------------------------------------------------------------------------

def _offsets(h: int) -> np.ndarray:
    return np.arange(-h, h + 1)


def _valid(L: int, h: int, active: np.ndarray | None) -> np.ndarray:
    """valid[k, i]: entry (i, i + k - h) lies in Omega and both tokens are active."""
    i = np.arange(L)[None, :]
    j = i + _offsets(h)[:, None]
    ok = (j >= 0) & (j < L)
    if active is not None:
        jc = np.clip(j, 0, L - 1)
        ok &= active[None, :] & active[jc]
    return ok


def _row_vec(v: np.ndarray, h: int) -> np.ndarray:
    """R[k, i] = v[i + k - h] (0 where the column index is out of range)."""
    L = v.shape[0]
    out = np.zeros((2 * h + 1, L))
    for k, o in enumerate(_offsets(h)):
        i0, i1 = max(0, -o), min(L, L - o)
        if i1 > i0:
            out[k, i0:i1] = v[i0 + o:i1 + o]
    return out


def _to_col(X: np.ndarray, h: int, fill: float) -> np.ndarray:
    """Xc[k, j] = X[k, j - (k - h)]: the same band entry indexed by its column."""
    L = X.shape[1]
    out = np.full_like(X, fill)
    for k, o in enumerate(_offsets(h)):
        j0, j1 = max(0, o), min(L, L + o)
        if j1 > j0:
            out[k, j0:j1] = X[k, j0 - o:j1 - o]
    return out


def _col_vec(u: np.ndarray, h: int) -> np.ndarray:
    """C[k, j] = u[j - (k - h)] (0 where the row index is out of range)."""
    L = u.shape[0]
    out = np.zeros((2 * h + 1, L))
    for k, o in enumerate(_offsets(h)):
        j0, j1 = max(0, o), min(L, L + o)
        if j1 > j0:
            out[k, j0:j1] = u[j0 - o:j1 - o]
    return out


def _neg_lse_axis0(X: np.ndarray) -> np.ndarray:
    """-log(sum_k exp(X[k, :])) with an exact max shift; an empty (all -inf) column
    gives 0, the convention for tokens that carry no mass (inactive fill tokens)."""
    m = X.max(axis=0)
    empty = ~np.isfinite(m)
    ms = np.where(empty, 0.0, m)
    with np.errstate(invalid="ignore"):
        tot = np.exp(X - ms[None, :]).sum(axis=0)
    out = -(ms + np.log(np.where(empty, 1.0, tot)))
    return np.where(empty, 0.0, out)


# --------------------------------------------------------------------------------------
# scores and dual updates
# --------------------------------------------------------------------------------------

def band_scores(Q: np.ndarray, K: np.ndarray, h: int, eps: float,
                active: np.ndarray | None = None) -> np.ndarray:
    """Scores on the fixed band support with the temperature absorbed:
    S_ij = q_i . k_j / (sqrt(d) * eps) for |i - j| <= h, -inf elsewhere.
    [technical summaries §2.1: fixed active support of band width W, epsilon absorbed
    into the score matrix S]"""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    L, d = Q.shape
    s = 1.0 / (np.sqrt(d) * eps)
    S = np.full((2 * h + 1, L), NEG_INF)
    for k, o in enumerate(_offsets(h)):
        i0, i1 = max(0, -o), min(L, L - o)
        if i1 > i0:
            S[k, i0:i1] = s * np.einsum("id,id->i", Q[i0:i1], K[i0 + o:i1 + o])
    S[~_valid(L, h, active)] = NEG_INF
    return S


def row_update(S: np.ndarray, v: np.ndarray, h: int) -> np.ndarray:
    """Balanced row half-step: u_i = -log sum_j exp(S_ij + v_j), so every row of
    exp(S + u + v) sums to 1 (unit row marginal).
    [abstract: balanced entropic OT; technical summaries §2.1: T-step balanced
    Sinkhorn iteration]"""
    return _neg_lse_axis0(S + _row_vec(v, h))


def col_update(S: np.ndarray, u: np.ndarray, h: int) -> np.ndarray:
    """Balanced column half-step: v_j = -log sum_i exp(S_ij + u_i), so every column
    of exp(S + u + v) sums to 1 (unit column marginal).  [same passages as row_update]"""
    return _neg_lse_axis0(_to_col(S, h, NEG_INF) + _col_vec(u, h))


def staircase_plan(S: np.ndarray, ua: np.ndarray, vb: np.ndarray, h: int) -> np.ndarray:
    """P^(a,b)_ij = exp(S_ij + u^(a)_i + v^(b)_j) on the band (0 off Omega).
    [technical summaries §2.2: the staircase plan factors]"""
    with np.errstate(invalid="ignore"):
        P = np.exp(S + ua[None, :] + _row_vec(vb, h))
    return np.where(np.isfinite(S), P, 0.0)


# --------------------------------------------------------------------------------------
# forward
# --------------------------------------------------------------------------------------

def _forward_duals(S: np.ndarray, h: int, T: int, R: int):
    """Stopped base followed by the refinement tail.

    Base: u = v = 0, then T steps of (row update, column update); the base result
    v^(0) is under stop-gradient.  Tail: for a = 1..R, u^(a) from v^(a-1), then
    v^(a) from u^(a).  Returns [v^(0), u^(1), v^(1), ..., u^(R), v^(R)].
    [technical summaries §2.1: stopped T-step base solve producing (u^(0), v^(0)),
    then R differentiable steps starting from the stopped base state]

    With R = 0 the output plan is the base's own, P^(0,0) = exp(S + u^(0) + v^(0)), and both
    of its duals are returned: [u^(0), v^(0)].  In every case the last two entries are the
    duals of the output plan."""
    L = S.shape[1]
    u = np.zeros(L)
    v = np.zeros(L)
    for _ in range(T):
        u = row_update(S, v, h)
        v = col_update(S, u, h)
    if R == 0:
        return [u.copy(), v.copy()]
    duals = [v.copy()]
    for _ in range(R):
        u = row_update(S, v, h)
        v = col_update(S, u, h)
        duals += [u.copy(), v.copy()]
    return duals


def forward(Q, K, V, prob: BandProblem, active=None):
    """Forward pass of one head: O = P^(R,R) V with P^(R,R) = exp(S + u^(R) + v^(R))
    on the band.  Returns (O, duals) with duals = [v0, u1, v1, ..., uR, vR].
    [technical summaries §2.1 (forward pass) and §2.2 (reference plan P^(2,2))]"""
    h = prob.h
    S = band_scores(Q, K, h, prob.eps, active)
    duals = _forward_duals(S, h, prob.T, prob.R)
    uR, vR = duals[-2], duals[-1]
    P = staircase_plan(S, uR, vR, h)
    V = np.asarray(V, dtype=np.float64)
    O = _band_matvec_rows(P, V, h)
    return O, np.stack(duals)


def forward_from_base(Q, K, V, v0, prob: BandProblem, active=None, u0=None):
    """Tail and output with the stopped base dual v^(0) supplied and held fixed:
    this is the function the tail VJP differentiates (v^(0) carries no gradient).
    R = 0 outputs with the base plan itself, so u^(0) is supplied and held fixed as well.
    [technical summaries §2.1: the tail refines the potentials starting from the
    stopped base state]"""
    h = prob.h
    S = band_scores(Q, K, h, prob.eps, active)
    v = np.asarray(v0, dtype=np.float64)
    if prob.R == 0 and u0 is None:
        raise ValueError("R = 0 differentiates with both base duals fixed: pass u0")
    u = None if u0 is None else np.asarray(u0, dtype=np.float64)
    for _ in range(prob.R):
        u = row_update(S, v, h)
        v = col_update(S, u, h)
    P = staircase_plan(S, u, v, h)
    return _band_matvec_rows(P, np.asarray(V, dtype=np.float64), h)


def _band_matvec_rows(X: np.ndarray, Y: np.ndarray, h: int) -> np.ndarray:
    """out_i = sum_j X_ij Y_j (row-indexed band X, rows of Y indexed by column j)."""
    L = X.shape[1]
    out = np.zeros((L, Y.shape[1]))
    for k, o in enumerate(_offsets(h)):
        i0, i1 = max(0, -o), min(L, L - o)
        if i1 > i0:
            out[i0:i1] += X[k, i0:i1, None] * Y[i0 + o:i1 + o]
    return out


def _band_matvec_cols(X: np.ndarray, Y: np.ndarray, h: int) -> np.ndarray:
    """out_j = sum_i X_ij Y_i (contraction over the row index of a row-indexed band)."""
    L = X.shape[1]
    out = np.zeros((L, Y.shape[1]))
    for k, o in enumerate(_offsets(h)):
        i0, i1 = max(0, -o), min(L, L - o)
        if i1 > i0:
            out[i0 + o:i1 + o] += X[k, i0:i1, None] * Y[i0:i1]
    return out


def _row_sum(X: np.ndarray) -> np.ndarray:
    return X.sum(axis=0)


def _col_sum(X: np.ndarray, h: int) -> np.ndarray:
    return _to_col(X, h, 0.0).sum(axis=0)


def _value_scores(dO, V, h, active):
    """g_ij = dO_i . V_j on the band (0 off Omega): the cotangent of the plan entry."""
    dO = np.asarray(dO, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L = dO.shape[0]
    g = np.zeros((2 * h + 1, L))
    for k, o in enumerate(_offsets(h)):
        i0, i1 = max(0, -o), min(L, L - o)
        if i1 > i0:
            g[k, i0:i1] = np.einsum("id,id->i", dO[i0:i1], V[i0 + o:i1 + o])
    g[~_valid(L, h, active)] = 0.0
    return g


def _score_contractions(dS, Q, K, P, dO, h, s):
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    dQ = s * _band_matvec_rows(dS, K, h)
    dK = s * _band_matvec_cols(dS, Q, h)
    dV = _band_matvec_cols(P, dO, h)
    return dQ, dK, dV


# --------------------------------------------------------------------------------------
# VJP, R = 2: direct four-plan form (reverse mode through the tail, step by step)
# --------------------------------------------------------------------------------------

def vjp_direct_four(Q, K, V, dO, duals, prob: BandProblem, active=None, want_parts=False):
    """Exact VJP of O = P^(2,2) V through the R = 2 tail with v^(0) stopped, written as
    reverse-mode differentiation of each tail step in turn, every staircase plan
    evaluated from its own exponential.

    Reverse order of the tail steps:
      O = P22 V:            dV = P22^T dO, dP22_ij = g_ij = dO_i . V_j
      P22 = exp(S+u2+v2):   dS += P22 g, du2 += rowsum(P22 g), dv2 += colsum(P22 g)
      v2 = -LSE_col(S+u2):  weights P22;  dS -= P22 dv2_j, du2 -= rowsum(P22 dv2_j)
      u2 = -LSE_row(S+v1):  weights P21;  dS -= P21 du2_i, dv1 = -colsum(P21 du2_i)
      v1 = -LSE_col(S+u1):  weights P11;  dS -= P11 dv1_j, du1 = -rowsum(P11 dv1_j)
      u1 = -LSE_row(S+v0):  weights P10;  dS -= P10 du1_i  (v0 is stopped)
      S = s Q K^T:          dQ = s dS K, dK = s dS^T Q
    [technical summaries §2.2: the direct exact R = 2 adjoint evaluates the four
    staircase plan factors P^(2,2), P^(2,1), P^(1,1), P^(1,0); atlas.scime.ai Key
    results: the direct-four/recompute adjoint]"""
    if prob.R != 2:
        raise ValueError("the four-plan adjoint is the R = 2 case")
    h = prob.h
    Qd = np.asarray(Q, dtype=np.float64)
    d = Qd.shape[1]
    s = 1.0 / (np.sqrt(d) * prob.eps)
    S = band_scores(Q, K, h, prob.eps, active)
    v0, u1, v1, u2, v2 = duals
    P22 = staircase_plan(S, u2, v2, h)
    P21 = staircase_plan(S, u2, v1, h)
    P11 = staircase_plan(S, u1, v1, h)
    P10 = staircase_plan(S, u1, v0, h)
    g = _value_scores(dO, V, h, active)

    dv2 = _col_sum(P22 * g, h)
    du2 = _row_sum(P22 * g) - _row_sum(P22 * _row_vec(dv2, h))
    dv1 = -_col_sum(P21 * du2[None, :], h)
    du1 = -_row_sum(P11 * _row_vec(dv1, h))
    dS = (P22 * g - P22 * _row_vec(dv2, h) - P21 * du2[None, :]
          - P11 * _row_vec(dv1, h) - P10 * du1[None, :])
    dQ, dK, dV = _score_contractions(dS, Q, K, P22, dO, h, s)
    if want_parts:
        return dQ, dK, dV, dict(dS=dS, du2=du2, dv2=dv2, du1=du1, dv1=dv1,
                                P22=P22, P21=P21, P11=P11, P10=P10, g=g, S=S)
    return dQ, dK, dV


# --------------------------------------------------------------------------------------
# VJP, R = 2: one-reference-tile form
# --------------------------------------------------------------------------------------

def vjp_one_reference(Q, K, V, dO, duals, prob: BandProblem, active=None, want_parts=False):
    """Exact R = 2 VJP with the one-reference-tile schedule: only P^(2,2) is
    exponentiated; the other staircase plans enter through vector factors
    exp(u^(a) - u^(2)) and exp(v^(b) - v^(2)).

    Vector cotangents (each a reduction of the reference tile):
      dv2_j = sum_i P22_ij g_ij
      du2_i = sum_j P22_ij (g_ij - dv2_j)
      dv1_j = -exp(v1_j - v2_j) sum_i P22_ij du2_i
      du1_i = -exp(u1_i - u2_i) sum_j P22_ij exp(v1_j - v2_j) dv1_j
    Modifier field and score cotangent:
      M_ij = g_ij - dv2_j - du2_i e^{dv1_j} - e^{du1_i} dv1_j e^{dv1_j} - du1_i e^{du1_i} e^{dv0_j}
      (with e^{du_a} = exp(u^(a) - u^(2)), e^{dv_b} = exp(v^(b) - v^(2))),  dS = P22 * M.
    [abstract (dS = P22 * M, with M formed from the tail's vector cotangents and the
    exp(u^(a) - u^(2)), exp(v^(b) - v^(2)) factors); technical summaries §2.2: orbit
    equation P^(a,b) = P^(2,2) * exp(u^(a)-u^(2)) * exp(v^(b)-v^(2))]"""
    if prob.R != 2:
        raise ValueError("the one-reference schedule here is the R = 2 case")
    h = prob.h
    Qd = np.asarray(Q, dtype=np.float64)
    d = Qd.shape[1]
    s = 1.0 / (np.sqrt(d) * prob.eps)
    S = band_scores(Q, K, h, prob.eps, active)
    v0, u1, v1, u2, v2 = duals
    P22 = staircase_plan(S, u2, v2, h)
    g = _value_scores(dO, V, h, active)

    eu1 = np.exp(u1 - u2)          # row factor of P^(1,*)
    ev1 = np.exp(v1 - v2)          # column factor of P^(*,1)
    ev0 = np.exp(v0 - v2)          # column factor of P^(*,0)

    dv2 = _col_sum(P22 * g, h)
    du2 = _row_sum(P22 * (g - _row_vec(dv2, h)))
    dv1 = -ev1 * _col_sum(P22 * du2[None, :], h)
    du1 = -eu1 * _row_sum(P22 * _row_vec(ev1 * dv1, h))

    A, B, C = du2, eu1, du1 * eu1                      # per-row vectors
    D, E, F, G = dv2, ev1, dv1 * ev1, ev0              # per-column vectors
    M = (g - _row_vec(D, h) - A[None, :] * _row_vec(E, h)
         - B[None, :] * _row_vec(F, h) - C[None, :] * _row_vec(G, h))
    dS = P22 * M
    dQ, dK, dV = _score_contractions(dS, Q, K, P22, dO, h, s)
    if want_parts:
        return dQ, dK, dV, dict(dS=dS, M=M, du2=du2, dv2=dv2, du1=du1, dv1=dv1,
                                P22=P22, g=g, S=S)
    return dQ, dK, dV


# --------------------------------------------------------------------------------------
# VJP, any tail depth R >= 0
# --------------------------------------------------------------------------------------

def _tail_duals(duals, R):
    """duals = [v0, u1, v1, ..., uR, vR] -> (us, vs) with us[a] = u^(a) (a >= 1), vs[b] = v^(b);
    for R = 0, duals = [u0, v0] -> ([u0], [v0])."""
    if R == 0:
        if len(duals) != 2:
            raise ValueError("expected the 2 base duals (u^(0), v^(0)) for R = 0")
        return [duals[0]], [duals[1]]
    if len(duals) != 2 * R + 1:
        raise ValueError("expected 2 R + 1 saved duals")
    us = [None] + [duals[2 * a - 1] for a in range(1, R + 1)]
    vs = [duals[2 * b] for b in range(R + 1)]
    return us, vs


def vjp_tail(Q, K, V, dO, duals, prob: BandProblem, active=None, want_parts=False):
    """Exact VJP of O = P^(R,R) V through an R-step tail (any R >= 0) with v^(0) stopped:
    reverse-mode differentiation of the tail steps in turn, last step first, every
    staircase plan P^(a,b) = exp(S + u^(a) + v^(b)) from its own exponential.

      O = P^(R,R) V:            dV = P^(R,R)^T dO,  g_ij = dO_i . V_j
      P^(R,R):                  dS = P g,  du^(R) = rowsum(P g),  dv^(R) = colsum(P g)
      for a = R, R-1, ..., 1:
        v^(a) = -LSE_col(S + u^(a))     (weights P^(a,a), columns sum to one)
            dS -= P^(a,a) dv^(a)_j,  du^(a) -= rowsum(P^(a,a) dv^(a)_j)
        u^(a) = -LSE_row(S + v^(a-1))   (weights P^(a,a-1), rows sum to one)
            dS -= P^(a,a-1) du^(a)_i,  dv^(a-1) -= colsum(P^(a,a-1) du^(a)_i)   (a > 1;
            v^(0) is stopped)
      dQ = s dS K,  dK = s dS^T Q
    R = 2 is the four-plan adjoint of vjp_direct_four.  R = 0: both duals of P = P^(0,0) are
    stopped, so no dual carries a cotangent and dS = P g.
    [technical summaries §2.1: R differentiable tail steps from the stopped base state;
    §2.2: the exact tail adjoint through the staircase plans]"""
    R = prob.R
    h = prob.h
    d = np.asarray(Q).shape[1]
    s = 1.0 / (np.sqrt(d) * prob.eps)
    S = band_scores(Q, K, h, prob.eps, active)
    us, vs = _tail_duals(duals, R)
    L = S.shape[1]
    P = staircase_plan(S, us[R], vs[R], h)
    g = _value_scores(dO, V, h, active)
    dS = P * g
    du = [None] + [np.zeros(L) for _ in range(R)]
    dv = [np.zeros(L) for _ in range(R + 1)]
    if R >= 1:
        du[R] = du[R] + _row_sum(P * g)
        dv[R] = dv[R] + _col_sum(P * g, h)
    for a in range(R, 0, -1):
        Paa = staircase_plan(S, us[a], vs[a], h)
        dS = dS - Paa * _row_vec(dv[a], h)
        du[a] = du[a] - _row_sum(Paa * _row_vec(dv[a], h))
        Pab = staircase_plan(S, us[a], vs[a - 1], h)
        dS = dS - Pab * du[a][None, :]
        if a > 1:
            dv[a - 1] = dv[a - 1] - _col_sum(Pab * du[a][None, :], h)
    dQ, dK, dV = _score_contractions(dS, Q, K, P, dO, h, s)
    if want_parts:
        return dQ, dK, dV, dict(dS=dS, du=du, dv=dv, P=P, g=g, S=S)
    return dQ, dK, dV


def vjp_tail_one_reference(Q, K, V, dO, duals, prob: BandProblem, active=None,
                           want_parts=False):
    """The same VJP (any R >= 0) with one reference tile: only P = P^(R,R) is
    exponentiated; every other staircase plan is P * eu_a(i) * ev_b(j) with
    eu_a = exp(u^(a) - u^(R)), ev_b = exp(v^(b) - v^(R)) (the orbit equation).

    Vector cotangents, each a reduction of the reference tile:
      dv^(R)_j = sum_i P_ij g_ij
      du^(R)_i = sum_j P_ij (g_ij - dv^(R)_j)
      for a = R-1, ..., 1:
        dv^(a)_j = -ev_a(j) sum_i P_ij eu_{a+1}(i) du^(a+1)_i
        du^(a)_i = -eu_a(i) sum_j P_ij ev_a(j) dv^(a)_j
    Modifier field (2 R rank-one terms) and score cotangent:
      M_ij = g_ij - sum_a eu_a(i) ev_a(j) dv^(a)_j - sum_a eu_a(i) du^(a)_i ev_{a-1}(j),
      dS = P * M.
    R = 2 is vjp_one_reference; R = 0 has no levels, so M = g.
    [abstract (dS = P^(R,R) * M, M of rank 2 R from the vector cotangents and the dual
    differences); technical summaries §2.2: orbit equation P^(a,b) = P^(R,R) exp(du) exp(dv)]"""
    R = prob.R
    h = prob.h
    d = np.asarray(Q).shape[1]
    s = 1.0 / (np.sqrt(d) * prob.eps)
    S = band_scores(Q, K, h, prob.eps, active)
    us, vs = _tail_duals(duals, R)
    P = staircase_plan(S, us[R], vs[R], h)
    g = _value_scores(dO, V, h, active)
    eu = [None] + [np.exp(us[a] - us[R]) for a in range(1, R + 1)]
    ev = [np.exp(vs[b] - vs[R]) for b in range(R + 1)]
    du = [None] * (R + 1)
    dv = [None] * (R + 1)
    dv[R] = _col_sum(P * g, h)
    du[R] = _row_sum(P * (g - _row_vec(dv[R], h)))
    for a in range(R - 1, 0, -1):
        dv[a] = -ev[a] * _col_sum(P * (eu[a + 1] * du[a + 1])[None, :], h)
        du[a] = -eu[a] * _row_sum(P * _row_vec(ev[a] * dv[a], h))
    M = g.copy()
    for a in range(1, R + 1):
        M = M - eu[a][None, :] * _row_vec(ev[a] * dv[a], h)
        M = M - (eu[a] * du[a])[None, :] * _row_vec(ev[a - 1], h)
    dS = P * M
    dQ, dK, dV = _score_contractions(dS, Q, K, P, dO, h, s)
    if want_parts:
        return dQ, dK, dV, dict(dS=dS, M=M, du=du, dv=dv, P=P, g=g, S=S)
    return dQ, dK, dV


# --------------------------------------------------------------------------------------
# full backpropagation and the a posteriori bias certificate
# --------------------------------------------------------------------------------------

def vjp_full(Q, K, V, dO, prob: BandProblem, active=None):
    """Exact gradient of <O, dO> through all T + R steps from u = v = 0, with no stop-gradient
    on the base: the same iteration read as a tail of depth T + R whose stopped base is the
    constant initial v = 0, differentiated step by step (vjp_tail).
    [technical summaries §2.4 and Key results: the stop-gradient surrogate compared with full
    backpropagation through time]"""
    pf = BandProblem(W=prob.W, T=0, R=prob.T + prob.R, eps=prob.eps)
    _, duals = forward(Q, K, V, pf, active)
    return vjp_tail(Q, K, V, dO, duals, pf, active)


def tail_remainder(Q, K, V, dO, prob: BandProblem, active=None) -> dict:
    """A posteriori bias certificate: the gradient remainder the stopped base drops at tail
    depth R, r = grad_full - grad_R, as squared norms summed over the tensor, and
    eta_R = ||(r_dQ, r_dK)|| / ||(dQ_full, dK_full)||.  dV has no remainder (V enters only the
    output), which the result reports as rem_dV2.
    [technical summaries §2.4: an operational measurement of the gradient remainder eta_R,
    certified against a user tolerance tau, selecting the tail depth R]"""
    _, duals = forward(Q, K, V, prob, active)
    fn = vjp_one_reference if prob.R == 2 else vjp_tail_one_reference
    dQr, dKr, dVr = fn(Q, K, V, dO, duals, prob, active)
    dQf, dKf, dVf = vjp_full(Q, K, V, dO, prob, active)
    out = {"rem_dQ2": float(np.sum((dQf - dQr) ** 2)), "full_dQ2": float(np.sum(dQf ** 2)),
           "rem_dK2": float(np.sum((dKf - dKr) ** 2)), "full_dK2": float(np.sum(dKf ** 2)),
           "rem_dV2": float(np.sum((dVf - dVr) ** 2))}
    den = out["full_dQ2"] + out["full_dK2"]
    out["eta"] = float(np.sqrt((out["rem_dQ2"] + out["rem_dK2"]) / den)) if den > 0 else 0.0
    return out


def select_tail_depth(Q, K, V, dO, W: int, T: int, eps: float = 1.0, tau: float = 1e-5,
                      R_max: int = 4, R_min: int = 0):
    """Smallest R in R_min..R_max with eta_R <= tau (None if none), and the eta_R computed.
    [technical summaries §2.4: dynamic choice of the tail depth; Key results: R = 2 is the
    smallest depth meeting tau = 1e-5 on the pages' problems]"""
    etas = {}
    for R in range(R_min, R_max + 1):
        etas[R] = tail_remainder(Q, K, V, dO, BandProblem(W=W, T=T, R=R, eps=eps))["eta"]
        if etas[R] <= tau:
            return R, etas
    return None, etas


# --------------------------------------------------------------------------------------
# dustbin_block: same surrogate on an augmented support
# --------------------------------------------------------------------------------------

def _augment(Xa: np.ndarray, block: int):
    """Append inactive fill tokens (zeros) so the token count is a multiple of `block`."""
    n = Xa.shape[0]
    Lp = -(-n // block) * block
    out = np.zeros((Lp, Xa.shape[1]))
    out[:n] = Xa
    return out


def _dustbin_setup(n_active: int, prob: BandProblem, block: int):
    Lp = -(-n_active // block) * block
    active = np.zeros(Lp, dtype=bool)
    active[:n_active] = True
    # widened band: every active token reaches the dustbin at index n_active - 1
    h_eff = max(prob.h, n_active - 1)
    return active, BandProblem(W=2 * h_eff, T=prob.T, R=prob.R, eps=prob.eps)


def dustbin_block_forward(Qa, Ka, Va, prob: BandProblem, block: int = 64):
    """dustbin_block forward.  Inputs hold L real tokens followed by one learned dustbin
    token (row L).  The token set is padded with inactive fill tokens to a multiple of
    `block`; the support is every pair of active tokens within the widened band
    (half-width max(W/2, L), so the dustbin row and column are fully connected);
    every active token has unit row and column target, the dustbin included.
    The unchanged balanced surrogate then runs on this augmented support.
    [technical summaries §2.3: dustbin token plus inactive fill tokens appended to
    Q/K/V, same balanced fixed-support tail surrogate on the larger state space;
    searcharxiv abstract: unit-target surrogate, single active dustbin;
    atlas.scime.ai Limitations: widened band cost O(L * max(W, L))]"""
    n = np.asarray(Qa).shape[0]
    active, p2 = _dustbin_setup(n, prob, block)
    O, duals = forward(_augment(np.asarray(Qa, np.float64), block),
                       _augment(np.asarray(Ka, np.float64), block),
                       _augment(np.asarray(Va, np.float64), block), p2, active)
    return O[:n], duals[:, :n]


def dustbin_block_vjp(Qa, Ka, Va, dOa, duals, prob: BandProblem, block: int = 64,
                      schedule: str = "one_reference"):
    """dustbin_block VJP: the same tail adjoint on the augmented support; returns
    gradients for all L + 1 tokens including the dustbin.  R = 2: the one-reference or
    four-plan adjoint; other R: the general-depth orbit form ("one_reference") or step form.
    [technical summaries §2.3: the exact R = 2 adjoint and the one-reference schedule
    carry over to the augmented state space unchanged]"""
    n = np.asarray(Qa).shape[0]
    active, p2 = _dustbin_setup(n, prob, block)
    Lp = active.shape[0]
    dfull = np.zeros((duals.shape[0], Lp))
    dfull[:, :n] = duals
    if prob.R == 2:
        fn = vjp_one_reference if schedule == "one_reference" else vjp_direct_four
    else:
        fn = vjp_tail_one_reference if schedule == "one_reference" else vjp_tail
    dQ, dK, dV = fn(_augment(np.asarray(Qa, np.float64), block),
                    _augment(np.asarray(Ka, np.float64), block),
                    _augment(np.asarray(Va, np.float64), block),
                    _augment(np.asarray(dOa, np.float64), block), dfull, p2, active)
    return dQ[:n], dK[:n], dV[:n]


# --------------------------------------------------------------------------------------
# exact evaluation of selected rows of a long sequence
# --------------------------------------------------------------------------------------

def dependency_radius(prob: BandProblem) -> int:
    """Token distance beyond which inputs cannot influence a row's outputs.

    On the band each half-step couples only tokens within h of each other, so a
    window cut changes values at most h further inward per half-step.  The forward
    takes 2(T+R) half-steps plus the output contraction; the VJP adds the chain
    dv^(R) -> du^(R) -> ... -> dv^(1) -> du^(1) -> dS -> dQ/dK (2 R + 1 more hops;
    five at R = 2).  Rows farther than (2(T+R) + 2R + 2) h from an artificial cut
    are therefore computed exactly; the radius below adds two hops and 16 tokens
    of margin (at R = 2 it is (2(T+R) + 8) h + 16)."""
    return (2 * (prob.T + prob.R) + 2 * prob.R + 4) * prob.h + 16


def sampled_rows(Q, K, V, dO, prob: BandProblem, rows, schedule: str = "one_reference"):
    """Exact O, dQ, dK, dV (fp64) at the requested rows of one long head, each computed
    on the window of tokens within dependency_radius of it (the sequence ends are real
    boundaries and are kept).  Returns dict name -> [len(rows), d]."""
    L = Q.shape[0]
    H = dependency_radius(prob)
    rows = np.asarray(rows, dtype=np.int64)
    out = {k: np.zeros((rows.shape[0], Q.shape[1])) for k in ("O", "dQ", "dK", "dV")}
    if prob.R == 2:
        fn = vjp_one_reference if schedule == "one_reference" else vjp_direct_four
    else:
        fn = vjp_tail_one_reference if schedule == "one_reference" else vjp_tail
    for n, r in enumerate(rows):
        a, b = max(0, int(r) - H), min(L, int(r) + H + 1)
        sl = slice(a, b)
        O, duals = forward(Q[sl], K[sl], V[sl], prob)
        dQ, dK, dV = fn(Q[sl], K[sl], V[sl], dO[sl], duals, prob)
        for k, X in (("O", O), ("dQ", dQ), ("dK", dK), ("dV", dV)):
            out[k][n] = X[int(r) - a]
    return out


def row_range(Q, K, V, dO, prob: BandProblem, start: int, stop: int,
              schedules=("one_reference",)):
    """Exact O, saved duals and, per adjoint schedule, dQ, dK, dV (fp64) of the rows
    [start, stop) of one long head, computed on the tokens within dependency_radius of that
    range (the sequence ends are real boundaries and are kept).  The forward runs once and each
    schedule's VJP reads its duals.  Returns {"O": [n, d], "duals": [n_d, n],
    schedule: {"dQ", "dK", "dV": [n, d]}} with n = stop - start."""
    L = Q.shape[0]
    if not 0 <= start <= stop <= L:
        raise ValueError("row range outside the sequence")
    H = dependency_radius(prob)
    a, b = max(0, start - H), min(L, stop + H)
    sl, keep = slice(a, b), slice(start - a, stop - a)
    O, duals = forward(Q[sl], K[sl], V[sl], prob)
    out = {"O": O[keep], "duals": duals[:, keep]}
    for schedule in schedules:
        if prob.R == 2:
            fn = vjp_one_reference if schedule == "one_reference" else vjp_direct_four
        else:
            fn = vjp_tail_one_reference if schedule == "one_reference" else vjp_tail
        dQ, dK, dV = fn(Q[sl], K[sl], V[sl], dO[sl], duals, prob)
        out[schedule] = {"dQ": dQ[keep], "dK": dK[keep], "dV": dV[keep]}
    return out
