"""Linear projection + cross-entropy loss and its input gradient.

TEST INFRASTRUCTURE ONLY (see the package docstring): the plain CPU oracle.

The last layer of the fine-tuned model ("LLM Fine-Tuning in 2026: Unsloth vs
QLoRA vs Liger-Kernel", section 3, the fused cross-entropy): hidden states
X [T, D] are projected by the frozen output head W [V, D] to logits over the
vocabulary and scored against integer targets.  The fused form exists to avoid
holding the whole [T, V] logit matrix; what it computes is the ordinary loss:

    z_t    = W x_t                                   (logits, V values)
    lse_t  = log sum_v exp(z_tv)
    l_t    = lse_t - z_t[target_t]                   (0 where target_t = ignore)
    n      = number of tokens whose target is not `ignore`
    loss   = (1/n) sum_t l_t                         (0 when n = 0)
    dX_t   = (1/n) sum_v (softmax(z_t)_v - [v = target_t]) W_v   (0 for ignored t)

Readings (the page names neither the reduction nor the ignore rule): the
mean over the tokens that carry a target, with the usual ignore value -100, as
a cross-entropy loss is ordinarily defined; with no such token the loss and
its gradient are zero.

Everything in float64 with no intermediate rounding; the matrix product and
the row reductions are the only library primitives.  The log-sum-exp is taken
after subtracting each row's maximum, which leaves its value unchanged and
keeps exp from overflowing.
"""
from __future__ import annotations

import numpy as np

from .qlora import as_f64

IGNORE_INDEX = -100


def linear_ce(X, W, targets, ignore_index: int = IGNORE_INDEX, want_grad: bool = True):
    """Returns (loss, token_loss [T], dX [T, D] or None), all float64.

    token_loss[t] is l_t (0 for ignored tokens); loss is their mean over the
    n tokens that carry a target.
    """
    X, W = as_f64(X), as_f64(W)
    targets = np.asarray(targets, np.int64)
    T, V = X.shape[0], W.shape[0]
    valid = targets != ignore_index
    n = int(valid.sum())
    Z = X @ W.T
    zmax = Z.max(axis=1) if V > 0 and T > 0 else np.zeros(T)
    E = np.exp(Z - zmax[:, None])
    S = E.sum(axis=1)
    lse = zmax + np.log(S)
    tgt = np.where(valid, targets, 0)
    z_t = Z[np.arange(T), tgt]
    token_loss = np.where(valid, lse - z_t, 0.0)
    loss = float(token_loss.sum() / n) if n > 0 else 0.0
    if not want_grad:
        return loss, token_loss, None
    G = E / S[:, None]
    G[np.arange(T), tgt] -= 1.0
    G[~valid] = 0.0
    dX = (G @ W) / n if n > 0 else np.zeros_like(X)
    return loss, token_loss, dX
