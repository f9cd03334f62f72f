"""Pins of the oracle's linear + cross-entropy (loss and dX).

* equal logits: a head whose V rows are all the same vector gives every
  token the loss log V and a zero gradient (closed form);
* a large-margin head: logits L for the target and 0 elsewhere give the
  loss log(1 + (V - 1) exp(-L)) per token (closed form);
* the same loss, per-token losses and gradient from PyTorch's CPU
  cross_entropy (mean reduction, ignore_index) with autograd in float64, a
  library routine independent of the oracle's own steps;
* central finite differences of the loss in X for dX;
* shift invariance: adding one vector u to every head row shifts each
  token's logits by the same amount, which changes neither the loss nor dX;
* ignored targets: they add nothing and the mean is over the rest; with every
  target ignored the loss and dX are zero.
"""
import numpy as np
import pytest
import torch

from oracle import linear_ce as olc


def _rand(T, D, V, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, D))
    W = rng.standard_normal((V, D)) * 0.3
    t = rng.integers(0, V, T)
    return X, W, t


def test_equal_logits_closed_form():
    T, D, V = 5, 8, 37
    rng = np.random.default_rng(1)
    X = rng.standard_normal((T, D))
    W = np.tile(rng.standard_normal(D), (V, 1))
    t = rng.integers(0, V, T)
    loss, tl, dX = olc.linear_ce(X, W, t)
    np.testing.assert_allclose(tl, np.full(T, np.log(V)), rtol=1e-14)
    assert abs(loss - np.log(V)) <= 1e-14 * np.log(V)
    assert np.max(np.abs(dX)) <= 1e-15


def test_large_margin_closed_form():
    T, V, L = 4, 9, 6.5
    D = V
    X = np.zeros((T, D))
    t = np.array([2, 0, 8, 5])
    X[np.arange(T), t] = L          # x_t = L e_target, W = I: z = L e_target
    W = np.eye(V)
    loss, tl, _ = olc.linear_ce(X, W, t)
    want = np.log1p((V - 1) * np.exp(-L))
    np.testing.assert_allclose(tl, np.full(T, want), rtol=1e-13)
    assert abs(loss - want) <= 1e-13 * want


@pytest.mark.parametrize("T,D,V,every", [(7, 16, 50, 0), (12, 8, 33, 4), (3, 5, 2, 0)])
def test_matches_torch_cross_entropy(T, D, V, every):
    X, W, t = _rand(T, D, V, 10 + T)
    if every:
        t[every - 1::every] = olc.IGNORE_INDEX
    loss, tl, dX = olc.linear_ce(X, W, t)
    Xt = torch.tensor(X, dtype=torch.float64, requires_grad=True)
    Z = Xt @ torch.tensor(W, dtype=torch.float64).T
    tt = torch.tensor(t, dtype=torch.int64)
    ref = torch.nn.functional.cross_entropy(Z, tt, ignore_index=olc.IGNORE_INDEX, reduction="mean")
    per = torch.nn.functional.cross_entropy(Z.detach(), tt, ignore_index=olc.IGNORE_INDEX, reduction="none")
    ref.backward()
    assert abs(loss - ref.item()) <= 1e-13 * abs(ref.item())
    np.testing.assert_allclose(tl, per.numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(dX, Xt.grad.numpy(), rtol=1e-11, atol=1e-15)


def test_finite_differences():
    T, D, V = 4, 6, 11
    X, W, t = _rand(T, D, V, 5)
    t[1] = olc.IGNORE_INDEX
    _, _, dX = olc.linear_ce(X, W, t)
    h = 1e-6
    for i in range(T):
        for d in range(D):
            Xp, Xm = X.copy(), X.copy()
            Xp[i, d] += h
            Xm[i, d] -= h
            fd = (olc.linear_ce(Xp, W, t, want_grad=False)[0] - olc.linear_ce(Xm, W, t, want_grad=False)[0]) / (2 * h)
            assert abs(fd - dX[i, d]) <= 1e-7 * max(1.0, abs(dX[i, d]))


def test_shift_invariance():
    T, D, V = 6, 10, 23
    X, W, t = _rand(T, D, V, 7)
    u = np.random.default_rng(8).standard_normal(D) * 2.0
    l1, tl1, d1 = olc.linear_ce(X, W, t)
    l2, tl2, d2 = olc.linear_ce(X, W + u[None, :], t)
    assert abs(l1 - l2) <= 1e-12 * abs(l1)
    np.testing.assert_allclose(tl1, tl2, rtol=1e-11)
    np.testing.assert_allclose(d1, d2, rtol=1e-10, atol=1e-14)


def test_ignored_tokens():
    T, D, V = 8, 6, 13
    X, W, t = _rand(T, D, V, 9)
    keep = np.array([0, 2, 3, 6])
    t2 = np.full(T, olc.IGNORE_INDEX)
    t2[keep] = t[keep]
    loss, tl, dX = olc.linear_ce(X, W, t2)
    l_sub, tl_sub, d_sub = olc.linear_ce(X[keep], W, t[keep])
    assert abs(loss - l_sub) <= 1e-14 * abs(l_sub)
    np.testing.assert_allclose(tl[keep], tl_sub, rtol=1e-14)
    assert np.all(tl[np.setdiff1d(np.arange(T), keep)] == 0.0)
    # the mean is over 4 tokens, not 8: the kept rows of dX match the subset's
    np.testing.assert_allclose(dX[keep], d_sub, rtol=1e-13, atol=1e-16)
    assert np.all(dX[np.setdiff1d(np.arange(T), keep)] == 0.0)
    loss0, tl0, dX0 = olc.linear_ce(X, W, np.full(T, olc.IGNORE_INDEX))
    assert loss0 == 0.0 and np.all(tl0 == 0.0) and np.all(dX0 == 0.0)
