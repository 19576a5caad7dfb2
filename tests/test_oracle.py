"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test names the fact that pins the oracle: a closed form, an independent
implementation (tests/independent.py), finite differences, or an invariant that
the mathematics of balanced Sinkhorn scaling fixes.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import sinkhorn_band as sb
from tests.independent import dense_autograd, dense_scores, textbook_sinkhorn

rng = np.random.default_rng(1234)


def _qkv(L, d=8, seed=0, scale=1.0):
    r = np.random.default_rng(seed)
    return [scale * r.standard_normal((L, d)) for _ in range(4)]


def _dense_from_band(X, h):
    """Expand diagonal band storage into a dense [L, L] matrix (0 off the band)."""
    L = X.shape[1]
    D = np.zeros((L, L))
    for k, o in enumerate(range(-h, h + 1)):
        for i in range(L):
            j = i + o
            if 0 <= j < L:
                D[i, j] = X[k, i]
    return D


# --------------------------------------------------------------------------------------
# forward iteration
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("L,W,T", [(7, 4, 3), (12, 22, 5), (30, 6, 9), (1, 4, 2), (9, 0, 2)])
def test_base_duals_match_textbook_sinkhorn(L, W, T):
    """Log-domain band updates == multiplicative Sinkhorn-Knopp on the masked matrix."""
    Q, K, _, _ = _qkv(L, seed=L + W)
    S, mask = dense_scores(Q, K, W, 0.7)
    A = np.where(mask, np.exp(S), 0.0)
    a, b = textbook_sinkhorn(A, T)
    prob = sb.BandProblem(W=W, T=T - 1, R=1, eps=0.7)   # T-1 base steps + 1 tail step = T steps
    _, duals = oracle.forward(Q, K, Q, prob)
    np.testing.assert_allclose(duals[1], np.log(a), rtol=0, atol=1e-12)
    np.testing.assert_allclose(duals[2], np.log(b), rtol=0, atol=1e-12)


def test_two_by_two_closed_form():
    """A positive 2x2 matrix scaled to unit marginals is [[p, 1-p], [1-p, p]] with
    p / (1 - p) = sqrt(kappa), kappa = A11 A22 / (A12 A21)."""
    Q = np.array([[1.0], [-0.5]])
    K = np.array([[0.8], [0.3]])
    prob = sb.BandProblem(W=2, T=200, R=2, eps=1.0)
    _, duals = oracle.forward(Q, K, Q, prob)
    S = sb.band_scores(Q, K, 1, 1.0)
    P = _dense_from_band(sb.staircase_plan(S, duals[3], duals[4], 1), 1)
    kappa = math.exp((1.0 - (-0.5)) * (0.8 - 0.3))
    p = math.sqrt(kappa) / (1.0 + math.sqrt(kappa))
    np.testing.assert_allclose(P, [[p, 1 - p], [1 - p, p]], atol=1e-14)


def test_zero_width_band_is_identity():
    """W = 0: the only support entries are the diagonal, so P = I, O = V, dV = dO and
    the score gradients vanish."""
    Q, K, V, dO = _qkv(11)
    prob = sb.BandProblem(W=0, T=4, R=2)
    O, duals = oracle.forward(Q, K, V, prob)
    np.testing.assert_allclose(O, V, atol=1e-14)
    for fn in (oracle.vjp_one_reference, oracle.vjp_direct_four):
        dQ, dK, dV = fn(Q, K, V, dO, duals, prob)
        np.testing.assert_allclose(dV, dO, atol=1e-14)
        assert np.abs(dQ).max() < 1e-13 and np.abs(dK).max() < 1e-13


@pytest.mark.parametrize("L,W", [(23, 6), (40, 14), (9, 30)])
def test_half_step_marginals(L, W):
    """Each half-step balances its own side exactly: rows of P^(1,0), P^(2,1) and
    columns of P^(1,1), P^(2,2) sum to 1."""
    Q, K, _, _ = _qkv(L, seed=3)
    h = W // 2
    prob = sb.BandProblem(W=W, T=2, R=2, eps=0.5)
    _, (v0, u1, v1, u2, v2) = oracle.forward(Q, K, Q, prob)
    S = sb.band_scores(Q, K, h, 0.5)
    D = lambda a, b: _dense_from_band(sb.staircase_plan(S, a, b, h), h)  # noqa: E731
    np.testing.assert_allclose(D(u1, v0).sum(1), 1, atol=1e-13)
    np.testing.assert_allclose(D(u2, v1).sum(1), 1, atol=1e-13)
    np.testing.assert_allclose(D(u1, v1).sum(0), 1, atol=1e-13)
    np.testing.assert_allclose(D(u2, v2).sum(0), 1, atol=1e-13)


def test_long_base_converges_to_doubly_stochastic():
    """With many base steps the reference plan's rows also sum to 1 (the band scaling
    problem has a unique doubly stochastic solution)."""
    Q, K, _, _ = _qkv(50, seed=5, scale=0.5)
    prob = sb.BandProblem(W=10, T=400, R=2)
    _, (v0, u1, v1, u2, v2) = oracle.forward(Q, K, Q, prob)
    S = sb.band_scores(Q, K, 5, 1.0)
    P = _dense_from_band(sb.staircase_plan(S, u2, v2, 5), 5)
    np.testing.assert_allclose(P.sum(1), 1, atol=1e-10)


def test_cross_ratio_and_orbit_identity():
    """Every staircase plan is a row/column rescaling of the reference plan, so
    (i) P^(a,b) = P^(2,2) * exp(u^(a)-u^(2)) * exp(v^(b)-v^(2)) entrywise and
    (ii) the cross ratio P_ij P_kl / (P_il P_kj) equals exp(S_ij + S_kl - S_il - S_kj)."""
    L, W = 20, 8
    h = W // 2
    Q, K, _, _ = _qkv(L, seed=7)
    prob = sb.BandProblem(W=W, T=1, R=2)
    _, (v0, u1, v1, u2, v2) = oracle.forward(Q, K, Q, prob)
    S = sb.band_scores(Q, K, h, 1.0)
    P22 = sb.staircase_plan(S, u2, v2, h)
    Sd, mask = dense_scores(Q, K, W, 1.0)
    for ua, vb in ((u2, v1), (u1, v1), (u1, v0)):
        direct = _dense_from_band(sb.staircase_plan(S, ua, vb, h), h)
        orbit = _dense_from_band(P22, h) * np.exp(ua - u2)[:, None] * np.exp(vb - v2)[None, :]
        np.testing.assert_allclose(direct, orbit, rtol=1e-13, atol=1e-16)
        i, k, j, l_ = 5, 6, 7, 8          # all four pairs lie on the band
        cr = direct[i, j] * direct[k, l_] / (direct[i, l_] * direct[k, j])
        np.testing.assert_allclose(cr, math.exp(Sd[i, j] + Sd[k, l_] - Sd[i, l_] - Sd[k, j]),
                                   rtol=1e-12)


# --------------------------------------------------------------------------------------
# VJP
# --------------------------------------------------------------------------------------

CASES = [
    # L, W, T, eps
    (1, 4, 2, 1.0),
    (5, 2, 0, 1.0),
    (6, 12, 1, 0.8),
    (17, 6, 15, 1.0),
    (24, 10, 3, 0.5),
    (33, 0, 2, 1.0),
    (40, 80, 15, 1.3),
]


@pytest.mark.parametrize("L,W,T,eps", CASES)
def test_forward_and_vjp_match_dense_autograd(L, W, T, eps):
    """Band oracle == dense torch-fp64 autograd through the same surrogate."""
    Q, K, V, dO = _qkv(L, seed=L * 31 + W)
    prob = sb.BandProblem(W=W, T=T, R=2, eps=eps)
    O, duals = oracle.forward(Q, K, V, prob)
    Or, dQr, dKr, dVr, dualsr = dense_autograd(Q, K, V, dO, W, T, 2, eps)
    np.testing.assert_allclose(O, Or, atol=1e-12)
    np.testing.assert_allclose(duals, dualsr, atol=1e-11)
    for fn in (oracle.vjp_one_reference, oracle.vjp_direct_four):
        dQ, dK, dV = fn(Q, K, V, dO, duals, prob)
        np.testing.assert_allclose(dQ, dQr, atol=1e-11)
        np.testing.assert_allclose(dK, dKr, atol=1e-11)
        np.testing.assert_allclose(dV, dVr, atol=1e-11)


def test_vjp_central_finite_differences():
    """<dQ, e_Q> + <dK, e_K> + <dV, e_V> equals the directional derivative of
    <O, dO> with v^(0) frozen (central differences, error O(delta^2))."""
    L, W = 26, 10
    Q, K, V, dO = _qkv(L, seed=11)
    prob = sb.BandProblem(W=W, T=4, R=2, eps=0.9)
    O, duals = oracle.forward(Q, K, V, prob)
    v0 = duals[0]
    dQ, dK, dV = oracle.vjp_one_reference(Q, K, V, dO, duals, prob)
    r = np.random.default_rng(2)
    for _ in range(3):
        eQ, eK, eV = (r.standard_normal(Q.shape) for _ in range(3))
        delta = 1e-5
        f = lambda t: float(np.sum(oracle.forward_from_base(  # noqa: E731
            Q + t * eQ, K + t * eK, V + t * eV, v0, prob) * dO))
        fd = (f(delta) - f(-delta)) / (2 * delta)
        an = float(np.sum(dQ * eQ) + np.sum(dK * eK) + np.sum(dV * eV))
        assert abs(fd - an) < 1e-7 * max(1.0, abs(an)), (fd, an)


def test_score_cotangent_invariants():
    """Row sums of dS vanish (a per-row shift of S changes no plan); column sums
    equal -sum_i P^(1,0)_ij du1_i (the cotangent the stop-gradient on v^(0) drops);
    dV = P22^T dO exactly."""
    L, W = 37, 12
    h = W // 2
    Q, K, V, dO = _qkv(L, seed=13)
    prob = sb.BandProblem(W=W, T=6, R=2)
    _, duals = oracle.forward(Q, K, V, prob)
    _, _, dV, parts = oracle.vjp_direct_four(Q, K, V, dO, duals, prob, want_parts=True)
    dS = _dense_from_band(parts["dS"], h)
    np.testing.assert_allclose(dS.sum(1), 0, atol=1e-13)
    P10 = _dense_from_band(parts["P10"], h)
    np.testing.assert_allclose(dS.sum(0), -(P10 * parts["du1"][:, None]).sum(0), atol=1e-13)
    P22 = _dense_from_band(parts["P22"], h)
    np.testing.assert_allclose(dV, P22.T @ dO, atol=1e-13)


def test_one_reference_equals_direct_four_entrywise():
    L, W = 45, 16
    Q, K, V, dO = _qkv(L, seed=17)
    prob = sb.BandProblem(W=W, T=2, R=2, eps=0.6)
    _, duals = oracle.forward(Q, K, V, prob)
    a = oracle.vjp_one_reference(Q, K, V, dO, duals, prob, want_parts=True)
    b = oracle.vjp_direct_four(Q, K, V, dO, duals, prob, want_parts=True)
    np.testing.assert_allclose(a[3]["dS"], b[3]["dS"], atol=1e-13)
    for x, y in zip(a[:3], b[:3]):
        np.testing.assert_allclose(x, y, atol=1e-13)


@pytest.mark.parametrize("L,W,R", [(45, 16, 2), (60, 200, 2), (50, 12, 1), (40, 20, 4)])
def test_vector_cotangents_of_the_last_level_through_O_and_dV(L, W, R):
    """The last tail level's vector cotangents are contractions the forward and dV already hold:
    dv^(R)_j = sum_i P_ij (dO_i . V_j) = V_j . dV_j with dV_j = sum_i P_ij dO_i, and the row
    sum sum_j P_ij (dO_i . V_j) = dO_i . O_i with O_i = sum_j P_ij V_j (P = P^(R,R); exact
    algebra, here at fp64 rounding).  The GPU passes take them this way; a transposed reduction
    (row sums for dv, say) would fail this."""
    Q, K, V, dO = _qkv(L, seed=23 + R)
    prob = sb.BandProblem(W=W, T=2, R=R, eps=0.8)
    O, duals = oracle.forward(Q, K, V, prob)
    if R == 2:
        _, _, dV, parts = oracle.vjp_one_reference(Q, K, V, dO, duals, prob, want_parts=True)
        dv, P, g = parts["dv2"], parts["P22"], parts["g"]
    else:
        _, _, dV, parts = oracle.vjp_tail(Q, K, V, dO, duals, prob, want_parts=True)
        dv, P, g = parts["dv"][-1], parts["P"], parts["g"]
    np.testing.assert_allclose(dv, np.einsum("jd,jd->j", V, dV), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sb._row_sum(P * g), np.einsum("id,id->i", dO, O),
                               rtol=1e-12, atol=1e-12)


def test_gauge_shift_of_stopped_base_is_a_no_op():
    """Centering the stopped dual (v0 -> v0 - c) changes no plan: u^(1) absorbs +c and
    every later v absorbs -c, so O and all gradients are unchanged."""
    L, W = 30, 10
    Q, K, V, dO = _qkv(L, seed=19)
    prob = sb.BandProblem(W=W, T=5, R=2)
    O, duals = oracle.forward(Q, K, V, prob)
    c = duals[0].mean()
    O2 = oracle.forward_from_base(Q, K, V, duals[0] - c, prob)
    np.testing.assert_allclose(O, O2, atol=1e-13)
    shifted = duals.copy()
    shifted[0] -= c
    shifted[1] += c
    shifted[2] -= c
    shifted[3] += c
    shifted[4] -= c
    g1 = oracle.vjp_one_reference(Q, K, V, dO, duals, prob)
    g2 = oracle.vjp_one_reference(Q, K, V, dO, shifted, prob)
    for x, y in zip(g1, g2):
        np.testing.assert_allclose(x, y, atol=1e-12)


# --------------------------------------------------------------------------------------
# dustbin_block
# --------------------------------------------------------------------------------------

def test_dustbin_block_equals_dense_surrogate_on_augmented_tokens():
    """The dustbin path with inactive fill tokens == the plain dense surrogate (no fill)
    on the L + 1 augmented tokens, checked against dense autograd too."""
    L, d = 21, 8
    Qa, Ka, Va, dOa = _qkv(L + 1, d=d, seed=23)
    prob = sb.BandProblem(W=4, T=6, R=2, eps=1.0)
    O, duals = oracle.dustbin_block_forward(Qa, Ka, Va, prob, block=16)
    Or, dQr, dKr, dVr, dualsr = dense_autograd(Qa, Ka, Va, dOa, 2 * L, 6, 2, 1.0)
    np.testing.assert_allclose(O, Or, atol=1e-12)
    np.testing.assert_allclose(duals, dualsr, atol=1e-11)
    for sched in ("one_reference", "direct_four"):
        dQ, dK, dV = oracle.dustbin_block_vjp(Qa, Ka, Va, dOa, duals, prob, block=16,
                                              schedule=sched)
        np.testing.assert_allclose(dQ, dQr, atol=1e-11)
        np.testing.assert_allclose(dK, dKr, atol=1e-11)
        np.testing.assert_allclose(dV, dVr, atol=1e-11)


def test_dustbin_column_carries_unit_mass():
    L = 30
    Qa, Ka, Va, _ = _qkv(L + 1, seed=29)
    prob = sb.BandProblem(W=4, T=3, R=2)
    _, duals = oracle.dustbin_block_forward(Qa, Ka, Va, prob, block=8)
    S = sb.band_scores(Qa, Ka, L, 1.0)
    P = _dense_from_band(sb.staircase_plan(S, duals[3], duals[4], L), L)
    assert abs(P[:, L].sum() - 1.0) < 1e-13


# --------------------------------------------------------------------------------------
# exact evaluation of rows of a long sequence
# --------------------------------------------------------------------------------------

def test_sampled_rows_equal_full_evaluation():
    L, W = 1400, 8
    Q, K, V, dO = _qkv(L, seed=31)
    prob = sb.BandProblem(W=W, T=3, R=2)
    O, duals = oracle.forward(Q, K, V, prob)
    dQ, dK, dV = oracle.vjp_one_reference(Q, K, V, dO, duals, prob)
    rows = [0, 3, 700, 1399]
    got = oracle.sampled_rows(Q, K, V, dO, prob, rows)
    assert oracle.dependency_radius(prob) < 700
    for name, X in (("O", O), ("dQ", dQ), ("dK", dK), ("dV", dV)):
        np.testing.assert_allclose(got[name], X[rows], atol=1e-13)


def test_row_ranges_tile_the_full_evaluation():
    """Contiguous row ranges, each evaluated on its own window, put together give the full
    evaluation of every output, every saved dual and both schedules' gradients; the ranges
    meet away from the sequence ends, so each window is cut on both sides."""
    L, W = 2000, 8
    Q, K, V, dO = _qkv(L, seed=32)
    prob = sb.BandProblem(W=W, T=3, R=2)
    O, duals = oracle.forward(Q, K, V, prob)
    ref = {s: fn(Q, K, V, dO, duals, prob) for s, fn in
           (("one_reference", oracle.vjp_one_reference), ("direct_four", oracle.vjp_direct_four))}
    cuts = [0, 450, 1200, 1201, 2000]
    assert oracle.dependency_radius(prob) < 450
    parts = [oracle.row_range(Q, K, V, dO, prob, a, b, ("one_reference", "direct_four"))
             for a, b in zip(cuts[:-1], cuts[1:])]
    np.testing.assert_allclose(np.concatenate([p["O"] for p in parts]), O, atol=1e-13)
    np.testing.assert_allclose(np.concatenate([p["duals"] for p in parts], axis=1), duals,
                               atol=1e-12)
    for s, (dQ, dK, dV) in ref.items():
        for name, X in (("dQ", dQ), ("dK", dK), ("dV", dV)):
            np.testing.assert_allclose(np.concatenate([p[s][name] for p in parts]), X, atol=1e-13)
    # the output reaches (2 (T + R) + 1) h tokens: a window cut one hop closer than that
    # moves the output row visibly
    short = prob.h * 2 * (prob.T + prob.R)
    assert short < oracle.dependency_radius(prob)
    O_cut, _ = oracle.forward(Q[:1000 + short + 1], K[:1000 + short + 1], V[:1000 + short + 1], prob)
    assert np.abs(O_cut[1000] - O[1000]).max() > 1e-10
