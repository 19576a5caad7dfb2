"""Pins of the oracle's projective contraction certificate (CPU only).

Delta is pinned against Birkhoff's definition by enumeration (tests/independent.py), closed forms
(a rank-one score block has diameter 0; a 2 x 2 block has |S00 + S11 - S01 - S10|), its gauge
invariance, the support test of each block pair against a dense mask, and the contraction it
certifies: the log-domain row and column half-steps of each active block shrink the
oscillation seminorm (the Hilbert metric in log coordinates) by at most tanh(Delta / 4).
"""

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from tests.independent import cross_ratio_diameter


def _qk(L, d=8, seed=0, scale=1.0):
    r = np.random.default_rng(seed)
    return scale * r.standard_normal((L, d)), scale * r.standard_normal((L, d))


def _blocks(n, B):
    return [(b * B, min(b * B + B, n)) for b in range(-(-n // B))]


@pytest.mark.parametrize("L,W,B,eps,dustbin", [
    (37, 20, 16, 1.0, False), (50, 64, 16, 0.7, False), (40, 200, 32, 1.3, False),
    (33, 8, 16, 1.0, True), (17, 0, 16, 1.0, False)])
def test_diameters_match_the_cross_ratio_definition(L, W, B, eps, dustbin):
    """Each active block's Delta equals Birkhoff's diameter of exp(S) on that block, found by
    enumerating all 2 x 2 minors; a block pair is active exactly when a dense support mask is
    all true on it."""
    Q, K = _qk(L, seed=L + W)
    prob = oracle.BandProblem(W=W, T=1, R=2, eps=eps)
    delta = oracle.block_diameters(Q, K, prob, B, dustbin=dustbin)
    h = max(W // 2, L - 1) if dustbin else W // 2
    i = np.arange(L)
    mask = np.abs(i[:, None] - i[None, :]) <= h
    S = Q @ K.T / (np.sqrt(Q.shape[1]) * eps)
    nb, m = oracle.block_layout(L, h, B)
    assert delta.shape == (nb, 2 * m + 1)
    blocks = _blocks(L, B)
    seen = 0
    for rb, (r0, r1) in enumerate(blocks):
        for cb, (c0, c1) in enumerate(blocks):
            active = bool(mask[r0:r1, c0:c1].all())
            o = cb - rb
            if abs(o) > m:
                assert not active
                continue
            got = delta[rb, o + m]
            if not active:
                assert got == -1.0
                continue
            seen += 1
            want = cross_ratio_diameter(np.exp(S[r0:r1, c0:c1]))
            assert abs(got - want) < 1e-12 * max(1.0, want), (rb, cb, got, want)
    assert seen > 0


def test_rank_one_block_has_diameter_zero_and_2x2_closed_form():
    """S_ij = a_i + b_j maps every ray to one ray (Delta = 0, kappa = 0); a 2 x 2 block has
    Delta = |S00 + S11 - S01 - S10|."""
    L, d = 20, 4
    r = np.random.default_rng(1)
    a, b = r.standard_normal(L), r.standard_normal(L)
    Q = np.zeros((L, d))
    K = np.zeros((L, d))
    Q[:, 0], Q[:, 1] = a, 1.0
    K[:, 0], K[:, 1] = 1.0, b
    delta = oracle.block_diameters(Q, K, oracle.BandProblem(W=100, T=1, R=2, eps=1.0), 16)
    act = delta[delta >= 0]
    assert act.size == 4 and np.all(np.abs(act) < 1e-14)
    np.testing.assert_allclose(oracle.contraction_coefficients(delta)[delta >= 0], 0.0, atol=1e-14)
    Q2, K2 = _qk(2, seed=2)
    S = Q2 @ K2.T / np.sqrt(8)
    delta2 = oracle.block_diameters(Q2, K2, oracle.BandProblem(W=2, T=1, R=2, eps=1.0), 16)
    assert delta2.shape == (1, 1)
    assert abs(delta2[0, 0] - abs(S[0, 0] + S[1, 1] - S[0, 1] - S[1, 0])) < 1e-14


def test_diameter_is_invariant_under_row_and_column_shifts():
    """Adding a_i to row i and b_j to column j of S (a diagonal scaling of the kernel) leaves
    every cross ratio, hence Delta, unchanged."""
    L, d = 45, 6
    Q, K = _qk(L, d, seed=3)
    r = np.random.default_rng(4)
    a, b = r.standard_normal(L), r.standard_normal(L)
    Qs = np.concatenate([Q, a[:, None], np.ones((L, 1))], axis=1)
    Ks = np.concatenate([K, np.ones((L, 1)), b[:, None]], axis=1)
    Q0 = np.concatenate([Q, np.zeros((L, 2))], axis=1)
    K0 = np.concatenate([K, np.zeros((L, 2))], axis=1)
    prob = oracle.BandProblem(W=40, T=1, R=2, eps=0.9)
    np.testing.assert_allclose(oracle.block_diameters(Qs, Ks, prob, 16),
                               oracle.block_diameters(Q0, K0, prob, 16), atol=1e-12)


def _osc(x):
    return float(x.max() - x.min())


@pytest.mark.parametrize("B,scale", [(16, 1.0), (32, 0.5), (16, 2.0)])
def test_half_steps_contract_by_the_certified_coefficient(B, scale):
    """Birkhoff-Hopf on each active block: for random dual pairs the row half-step
    u = -logsumexp(S + v) and the column half-step shrink the oscillation of the difference by
    at most kappa = tanh(Delta / 4) < 1, and a full step by kappa^2."""
    L, W, eps = 70, 80, 1.0
    Q, K = _qk(L, seed=B + int(10 * scale), scale=scale)
    prob = oracle.BandProblem(W=W, T=1, R=2, eps=eps)
    delta = oracle.block_diameters(Q, K, prob, B)
    kappa = oracle.contraction_coefficients(delta)
    S = Q @ K.T / (np.sqrt(Q.shape[1]) * eps)
    nb, m = delta.shape[0], (delta.shape[1] - 1) // 2
    blocks = _blocks(L, B)
    r = np.random.default_rng(5)
    checked = 0
    for rb in range(nb):
        for o in range(-m, m + 1):
            if delta[rb, o + m] < 0:
                continue
            (r0, r1), (c0, c1) = blocks[rb], blocks[rb + o]
            Sb = S[r0:r1, c0:c1]
            k = kappa[rb, o + m]
            assert 0.0 <= k < 1.0
            for _ in range(20):
                v1, v2 = 3 * r.standard_normal(c1 - c0), 3 * r.standard_normal(c1 - c0)
                u1, u2 = -logsumexp(Sb + v1[None, :], axis=1), -logsumexp(Sb + v2[None, :], axis=1)
                assert _osc(u1 - u2) <= k * _osc(v1 - v2) + 1e-12
                w1, w2 = -logsumexp(Sb.T + u1[None, :], axis=1), -logsumexp(Sb.T + u2[None, :], axis=1)
                assert _osc(w1 - w2) <= k * k * _osc(v1 - v2) + 1e-12
            checked += 1
    assert checked >= nb


def test_dense_dustbin_support_makes_every_block_active():
    L = 40
    Q, K = _qk(L + 1, seed=6)
    delta = oracle.block_diameters(Q, K, oracle.BandProblem(W=4, T=1, R=2, eps=1.0), 16,
                                   dustbin=True)
    assert delta.shape == (3, 5)
    for rb in range(3):
        for o in range(-2, 3):
            assert (delta[rb, o + 2] >= 0) == (0 <= rb + o < 3)
