"""RMSNorm forward and hand-derived backward.

TEST INFRASTRUCTURE ONLY (see the package docstring): the plain CPU oracle.

The normalisation in front of the MLP block ("LLM Fine-Tuning in 2026:
Unsloth vs QLoRA vs Liger-Kernel", the fused-RMSNorm part of section 2: the
forward keeps only one inverse RMS per row for the backward instead of any
full-size intermediate).  Per row x of D elements, weight w [D], eps > 0:

    ms   = (1/D) sum_j x_j^2
    rstd = 1 / sqrt(ms + eps)                 (saved, one float per row)
    y    = x * rstd * w

Backward of the loss <Y, dY> (derived here; the pages only say it is derived
by hand), with g = dy * w:

    dx = rstd * g - (rstd^3 / D) * (sum_j g_j x_j) * x
    dw = sum over rows of dy * x * rstd

Everything in float64 with no intermediate rounding; matrix and row sums are
the only library primitives.
"""
from __future__ import annotations

import numpy as np

from .qlora import as_f64


def rmsnorm_forward(X, w, eps: float):
    """Returns (Y, rstd) in float64: Y [M, D], rstd [M]."""
    X, w = as_f64(X), as_f64(w)
    ms = np.mean(X * X, axis=1)
    rstd = 1.0 / np.sqrt(ms + eps)
    return X * rstd[:, None] * w[None, :], rstd


def rmsnorm_backward(dY, X, w, rstd):
    """Gradients of <Y, dY> given the saved rstd: returns (dX, dw) in float64."""
    dY, X, w, rstd = as_f64(dY), as_f64(X), as_f64(w), np.asarray(rstd, np.float64)
    D = X.shape[1]
    g = dY * w[None, :]
    c = np.sum(g * X, axis=1)
    dX = rstd[:, None] * g - (rstd ** 3 / D * c)[:, None] * X
    dw = np.sum(dY * X * rstd[:, None], axis=0)
    return dX, dw
