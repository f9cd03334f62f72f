"""Pins of the oracle's RMSNorm.

* forward: a constant row c has mean square c^2, so y = c w / sqrt(c^2 + eps)
  (closed form); scaling a row by lambda leaves y unchanged when eps = 0; the
  mean of (y / w)^2 over a row is ms / (ms + eps);
* backward: central finite differences of <Y, dY> in X and w, and the
  backward's dX is orthogonal-ish in the eps -> 0 limit: sum_j x_j dx_j = 0
  when eps = 0 and w = 1 (Y does not change along x).
"""
import numpy as np

from oracle import rmsnorm


def test_constant_row_closed_form():
    D, eps = 64, 1e-3
    w = np.linspace(-2.0, 3.0, D)
    for c in (0.0, 0.5, -3.0):
        Y, r = rmsnorm.rmsnorm_forward(np.full((1, D), c), w, eps)
        assert abs(r[0] - 1.0 / np.sqrt(c * c + eps)) <= 1e-15 * r[0]
        np.testing.assert_allclose(Y[0], c * w / np.sqrt(c * c + eps), rtol=1e-14, atol=1e-300)


def test_scale_invariance_without_eps():
    rng = np.random.default_rng(3)
    X, w = rng.standard_normal((5, 48)), rng.standard_normal(48)
    Y1, _ = rmsnorm.rmsnorm_forward(X, w, 0.0)
    Y2, _ = rmsnorm.rmsnorm_forward(X * 7.25, w, 0.0)
    np.testing.assert_allclose(Y1, Y2, rtol=1e-13)


def test_mean_square_of_normalised_row():
    rng = np.random.default_rng(4)
    X, eps = rng.standard_normal((6, 40)), 0.3
    Y, _ = rmsnorm.rmsnorm_forward(X, np.ones(40), eps)
    ms = np.mean(X * X, axis=1)
    np.testing.assert_allclose(np.mean(Y * Y, axis=1), ms / (ms + eps), rtol=1e-13)


def _loss(X, w, dY, eps):
    return float(np.sum(rmsnorm.rmsnorm_forward(X, w, eps)[0] * dY))


def test_backward_finite_differences():
    rng = np.random.default_rng(8)
    M, D, eps = 3, 16, 0.05
    X, w, dY = rng.standard_normal((M, D)), rng.standard_normal(D), rng.standard_normal((M, D))
    _, r = rmsnorm.rmsnorm_forward(X, w, eps)
    dX, dw = rmsnorm.rmsnorm_backward(dY, X, w, r)
    h = 1e-6
    for P, G in ((X, dX), (w, dw)):
        fd = np.zeros_like(P)
        for idx in np.ndindex(P.shape):
            old = P[idx]
            P[idx] = old + h
            fp = _loss(X, w, dY, eps)
            P[idx] = old - h
            fm = _loss(X, w, dY, eps)
            P[idx] = old
            fd[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(G, fd, rtol=1e-6, atol=1e-8)


def test_backward_orthogonal_to_row_without_eps():
    rng = np.random.default_rng(12)
    X, dY = rng.standard_normal((4, 32)), rng.standard_normal((4, 32))
    _, r = rmsnorm.rmsnorm_forward(X, np.ones(32), 0.0)
    dX, _ = rmsnorm.rmsnorm_backward(dY, X, np.ones(32), r)
    np.testing.assert_allclose(np.sum(X * dX, axis=1), 0.0, atol=1e-12)
