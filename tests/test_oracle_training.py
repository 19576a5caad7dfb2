"""Pins of the oracle's synthetic training step (CPU only).

The step's loss and weight gradients are pinned against torch float64 autograd through an
independent dense model with the same stopped-base surrogate (tests/independent.py), and against
central finite differences of the loss with every head's stopped base held fixed; the SGD update
is the gradient step it states.
"""

import numpy as np
import pytest

import oracle
from tests.independent import dense_reconstruction_grads


def _problem(B, L, D, seed, frac=0.25):
    r = np.random.default_rng(seed)
    X = r.standard_normal((B, L, D))
    mask = (r.random((B, L)) < frac).astype(np.float64)
    mask[:, 0] = 1.0
    params = tuple(r.standard_normal((D, D)) / np.sqrt(D) for _ in range(4))
    return params, X, mask


@pytest.mark.parametrize("B,L,D,H,W,T,R,eps", [
    (2, 24, 16, 2, 8, 3, 2, 1.0), (1, 30, 24, 3, 12, 4, 1, 0.8), (2, 20, 8, 1, 40, 2, 0, 1.0),
    (1, 18, 16, 2, 6, 2, 3, 1.2)])
def test_step_matches_dense_autograd(B, L, D, H, W, T, R, eps):
    params, X, mask = _problem(B, L, D, seed=L + D + R)
    cfg = oracle.TrainConfig(heads=H, W=W, T=T, R=R, eps=eps, lr=0.05)
    loss, grads, new = oracle.reconstruction_step(params, X, mask, cfg)
    loss_r, grads_r = dense_reconstruction_grads(params, X, mask, H, W, T, R, eps)
    assert abs(loss - loss_r) < 1e-12 * max(1.0, loss_r)
    for g, gr in zip(grads, grads_r):
        np.testing.assert_allclose(g, gr, atol=1e-11, rtol=0)
    for w, g, wn in zip(params, grads, new):
        np.testing.assert_allclose(wn, w - 0.05 * g, atol=0, rtol=0)


def test_step_gradient_central_finite_differences():
    """<grad, E> equals the directional derivative of the loss along E with each head's stopped
    base held at its saved duals."""
    params, X, mask = _problem(2, 22, 16, seed=9)
    cfg = oracle.TrainConfig(heads=2, W=10, T=3, R=2, eps=0.9)
    _, grads, _, duals = oracle.reconstruction_step(params, X, mask, cfg, want_duals=True)
    r = np.random.default_rng(10)
    for _ in range(2):
        E = [r.standard_normal(w.shape) for w in params]
        delta = 1e-5
        f = lambda t: oracle.reconstruction_loss(  # noqa: E731
            [w + t * e for w, e in zip(params, E)], X, mask, cfg, base=duals)
        fd = (f(delta) - f(-delta)) / (2 * delta)
        an = sum(float(np.sum(g * e)) for g, e in zip(grads, E))
        assert abs(fd - an) < 1e-7 * max(1.0, abs(an)), (fd, an)
    assert abs(oracle.reconstruction_loss(params, X, mask, cfg) -
               oracle.reconstruction_loss(params, X, mask, cfg, base=duals)) < 1e-14


def test_unmasked_tokens_do_not_enter_the_loss():
    """Changing X at unmasked tokens changes the loss only through the input projections: with
    the output projection zero the loss is the masked tokens' mean square, whatever X elsewhere."""
    params, X, mask = _problem(1, 16, 8, seed=11)
    params = params[:3] + (np.zeros((8, 8)),)
    cfg = oracle.TrainConfig(heads=1, W=6, T=2, R=2)
    loss, grads, _ = oracle.reconstruction_step(params, X, mask, cfg)
    want = float(np.sum((X * mask[..., None]) ** 2) / (mask.sum() * 8))
    assert abs(loss - want) < 1e-14
    for g in grads[:3]:
        np.testing.assert_allclose(g, 0.0, atol=1e-15)
