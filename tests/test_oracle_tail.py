"""Pins of the oracle's adjoint for a general tail depth R (CPU only).

The two general-R forms (step-by-step reverse mode with every staircase plan from its own
exponential, and the one-reference-tile orbit form) are pinned against dense torch fp64
autograd through the same surrogate (tests/independent.py), against central finite
differences with the stopped base held fixed, against the invariants that fix row and column
sums of the score cotangent, and, at R = 2, against the four-plan and one-reference functions.
"""

import numpy as np
import pytest

import oracle
from oracle import sinkhorn_band as sb
from tests.independent import dense_autograd


def _qkv(L, d=8, seed=0):
    r = np.random.default_rng(seed)
    return [r.standard_normal((L, d)) for _ in range(4)]


def _dense_from_band(X, h):
    L = X.shape[1]
    D = np.zeros((L, L))
    for k, o in enumerate(range(-h, h + 1)):
        for i in range(L):
            j = i + o
            if 0 <= j < L:
                D[i, j] = X[k, i]
    return D


CASES = [
    # L, W, T, R, eps
    (21, 8, 3, 1, 1.0),
    (30, 12, 0, 1, 0.7),
    (27, 10, 4, 3, 1.0),
    (40, 80, 5, 3, 1.2),
    (33, 14, 2, 4, 0.8),
    (18, 0, 1, 4, 1.0),
    (25, 10, 3, 0, 1.0),
    (20, 40, 1, 0, 0.8),
]


@pytest.mark.parametrize("L,W,T,R,eps", CASES)
def test_tail_vjp_matches_dense_autograd(L, W, T, R, eps):
    """Both general-R forms == dense torch-fp64 autograd through the same surrogate."""
    Q, K, V, dO = _qkv(L, seed=L * 7 + R)
    prob = sb.BandProblem(W=W, T=T, R=R, eps=eps)
    O, duals = oracle.forward(Q, K, V, prob)
    Or, dQr, dKr, dVr, dualsr = dense_autograd(Q, K, V, dO, W, T, R, eps)
    np.testing.assert_allclose(O, Or, atol=1e-12)
    np.testing.assert_allclose(duals, dualsr, atol=1e-11)
    for fn in (oracle.vjp_tail, oracle.vjp_tail_one_reference):
        dQ, dK, dV = fn(Q, K, V, dO, duals, prob)
        np.testing.assert_allclose(dQ, dQr, atol=1e-10)
        np.testing.assert_allclose(dK, dKr, atol=1e-10)
        np.testing.assert_allclose(dV, dVr, atol=1e-11)


def test_tail_forms_reduce_to_the_r2_adjoints():
    """At R = 2 the step-by-step form is the four-plan adjoint and the orbit form is the
    one-reference adjoint, entry by entry."""
    L, W = 35, 12
    Q, K, V, dO = _qkv(L, seed=5)
    prob = sb.BandProblem(W=W, T=3, R=2, eps=0.9)
    _, duals = oracle.forward(Q, K, V, prob)
    a = oracle.vjp_tail(Q, K, V, dO, duals, prob, want_parts=True)
    b = oracle.vjp_direct_four(Q, K, V, dO, duals, prob, want_parts=True)
    c = oracle.vjp_tail_one_reference(Q, K, V, dO, duals, prob, want_parts=True)
    e = oracle.vjp_one_reference(Q, K, V, dO, duals, prob, want_parts=True)
    np.testing.assert_allclose(a[3]["dS"], b[3]["dS"], atol=1e-13)
    np.testing.assert_allclose(c[3]["dS"], e[3]["dS"], atol=1e-13)
    np.testing.assert_allclose(a[3]["du"][1], b[3]["du1"], atol=1e-13)
    np.testing.assert_allclose(c[3]["dv"][1], e[3]["dv1"], atol=1e-13)


@pytest.mark.parametrize("R", [1, 3, 4])
def test_tail_orbit_form_equals_step_form_entrywise(R):
    """Orbit identity: every staircase plan is the reference tile times row and column
    factors, so the two forms give the same score cotangent entry by entry."""
    L, W = 44, 14
    Q, K, V, dO = _qkv(L, seed=20 + R)
    prob = sb.BandProblem(W=W, T=2, R=R, eps=0.6)
    _, duals = oracle.forward(Q, K, V, prob)
    a = oracle.vjp_tail(Q, K, V, dO, duals, prob, want_parts=True)
    b = oracle.vjp_tail_one_reference(Q, K, V, dO, duals, prob, want_parts=True)
    np.testing.assert_allclose(a[3]["dS"], b[3]["dS"], atol=1e-13)
    for a_ in range(1, R + 1):
        np.testing.assert_allclose(a[3]["du"][a_], b[3]["du"][a_], atol=1e-13)
        np.testing.assert_allclose(a[3]["dv"][a_], b[3]["dv"][a_], atol=1e-13)


@pytest.mark.parametrize("R", [1, 4])
def test_tail_invariants(R):
    """Row sums of dS vanish (the tail starts with a row update, which absorbs a per-row
    shift of S); column sums equal -sum_i P^(1,0)_ij du^(1)_i, the cotangent of the stopped
    v^(0); dV = P^(R,R)^T dO."""
    L, W = 31, 10
    h = W // 2
    Q, K, V, dO = _qkv(L, seed=40 + R)
    prob = sb.BandProblem(W=W, T=3, R=R)
    _, duals = oracle.forward(Q, K, V, prob)
    _, _, dV, parts = oracle.vjp_tail(Q, K, V, dO, duals, prob, want_parts=True)
    dS = _dense_from_band(parts["dS"], h)
    np.testing.assert_allclose(dS.sum(1), 0, atol=1e-13)
    P10 = _dense_from_band(sb.staircase_plan(parts["S"], duals[1], duals[0], h), h)
    np.testing.assert_allclose(dS.sum(0), -(P10 * parts["du"][1][:, None]).sum(0), atol=1e-13)
    P = _dense_from_band(parts["P"], h)
    np.testing.assert_allclose(dV, P.T @ dO, atol=1e-13)


def test_r0_is_the_stopped_base_plan():
    """R = 0 outputs with the base's own plan: the same iterates as one tail step after T - 1
    base steps, so O and the plan's duals agree with (T - 1, R = 1); with both duals stopped,
    dS = P g and dV = P^T dO."""
    L, W, T = 29, 10, 4
    h = W // 2
    Q, K, V, dO = _qkv(L, seed=90)
    p0 = sb.BandProblem(W=W, T=T, R=0, eps=0.9)
    p1 = sb.BandProblem(W=W, T=T - 1, R=1, eps=0.9)
    O0, d0 = oracle.forward(Q, K, V, p0)
    O1, d1 = oracle.forward(Q, K, V, p1)
    assert d0.shape == (2, L)
    np.testing.assert_allclose(O0, O1, atol=1e-14)
    np.testing.assert_allclose(d0, d1[1:], atol=1e-14)
    _, _, dV, parts = oracle.vjp_tail(Q, K, V, dO, d0, p0, want_parts=True)
    P = _dense_from_band(parts["P"], h)
    G = dO @ V.T
    np.testing.assert_allclose(_dense_from_band(parts["dS"], h), P * G, atol=1e-13)
    np.testing.assert_allclose(dV, P.T @ dO, atol=1e-13)
    with pytest.raises(ValueError):
        sb.BandProblem(W=W, T=0, R=0)


def test_r0_central_finite_differences():
    """R = 0: the VJP is the derivative of <O, dO> with u^(0) and v^(0) both frozen."""
    L, W = 22, 8
    Q, K, V, dO = _qkv(L, seed=91)
    prob = sb.BandProblem(W=W, T=3, R=0, eps=0.8)
    _, duals = oracle.forward(Q, K, V, prob)
    dQ, dK, dV = oracle.vjp_tail_one_reference(Q, K, V, dO, duals, prob)
    r = np.random.default_rng(5)
    for _ in range(3):
        eQ, eK, eV = (r.standard_normal(Q.shape) for _ in range(3))
        delta = 1e-5
        f = lambda t: float(np.sum(oracle.forward_from_base(  # noqa: E731
            Q + t * eQ, K + t * eK, V + t * eV, duals[1], prob, u0=duals[0]) * dO))
        fd = (f(delta) - f(-delta)) / (2 * delta)
        an = float(np.sum(dQ * eQ) + np.sum(dK * eK) + np.sum(dV * eV))
        assert abs(fd - an) < 1e-7 * max(1.0, abs(an)), (fd, an)


def test_tail_vjp_central_finite_differences():
    """R = 4: <dQ, e_Q> + <dK, e_K> + <dV, e_V> equals the directional derivative of
    <O, dO> with v^(0) frozen (central differences)."""
    L, W = 24, 8
    Q, K, V, dO = _qkv(L, seed=3)
    prob = sb.BandProblem(W=W, T=3, R=4, eps=0.9)
    _, duals = oracle.forward(Q, K, V, prob)
    v0 = duals[0]
    dQ, dK, dV = oracle.vjp_tail_one_reference(Q, K, V, dO, duals, prob)
    r = np.random.default_rng(4)
    for _ in range(3):
        eQ, eK, eV = (r.standard_normal(Q.shape) for _ in range(3))
        delta = 1e-5
        f = lambda t: float(np.sum(oracle.forward_from_base(  # noqa: E731
            Q + t * eQ, K + t * eK, V + t * eV, v0, prob) * dO))
        fd = (f(delta) - f(-delta)) / (2 * delta)
        an = float(np.sum(dQ * eQ) + np.sum(dK * eK) + np.sum(dV * eV))
        assert abs(fd - an) < 1e-7 * max(1.0, abs(an)), (fd, an)


# --------------------------------------------------------------------------------------
# full backpropagation and the a posteriori bias certificate
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("L,W,T,R,eps", [(22, 8, 3, 2, 1.0), (30, 12, 5, 1, 0.8), (26, 60, 4, 3, 1.1),
                                         (24, 10, 3, 0, 0.9)])
def test_full_backprop_matches_dense_autograd_through_the_base(L, W, T, R, eps):
    """vjp_full == dense autograd with gradients flowing through every base step."""
    from tests.independent import dense_autograd_full
    Q, K, V, dO = _qkv(L, seed=60 + L)
    prob = sb.BandProblem(W=W, T=T, R=R, eps=eps)
    _, dQr, dKr, dVr = dense_autograd_full(Q, K, V, dO, W, T, R, eps)
    dQ, dK, dV = oracle.vjp_full(Q, K, V, dO, prob)
    np.testing.assert_allclose(dQ, dQr, atol=1e-10)
    np.testing.assert_allclose(dK, dKr, atol=1e-10)
    np.testing.assert_allclose(dV, dVr, atol=1e-11)


def test_remainder_invariants():
    """No dV remainder (V enters only the output); no remainder at all without a base (T = 0:
    the stopped v^(0) = 0 is a constant); the remainder at R is the gradient the tail drops,
    nonzero for T > 0."""
    L, W = 28, 10
    Q, K, V, dO = _qkv(L, seed=70)
    r = oracle.tail_remainder(Q, K, V, dO, sb.BandProblem(W=W, T=4, R=2, eps=0.8))
    assert r["rem_dV2"] < 1e-24 * max(1.0, r["full_dQ2"])
    assert r["eta"] > 1e-8
    r0 = oracle.tail_remainder(Q, K, V, dO, sb.BandProblem(W=W, T=0, R=3, eps=0.8))
    assert r0["eta"] < 1e-13


def test_remainder_decays_with_tail_depth():
    """The bias of the stopped base shrinks as the tail deepens (the refinement map contracts,
    technical summaries §2.4; Key results, bias decay from R = 0 through 1 and 2): eta_R
    decreases strictly from R = 0 to 4 on a base far from converged."""
    L, W = 40, 12
    Q, K, V, dO = _qkv(L, seed=71)
    etas = [oracle.tail_remainder(Q, K, V, dO, sb.BandProblem(W=W, T=2, R=R, eps=1.0))["eta"]
            for R in (0, 1, 2, 3, 4)]
    assert all(b < a for a, b in zip(etas, etas[1:])), etas


def test_select_tail_depth_returns_the_smallest_certified_depth():
    """On a strongly contracting problem (dense support, low-contrast scores) the remainder
    falls by about three decades per tail step and R = 2 is the smallest depth certified at
    tau = 1e-5 (the selection the pages report, Key results); the selection stops there."""
    r = np.random.default_rng(72)
    Q, K, V, dO = (r.standard_normal((64, 64)) for _ in range(4))
    Q, K = 0.3 * Q, 0.3 * K
    R, etas = oracle.select_tail_depth(Q, K, V, dO, W=128, T=15, eps=1.0, tau=1e-5, R_max=4)
    assert R == 2, etas
    assert etas[0] > etas[1] > 1e-5 >= etas[2] and 3 not in etas
