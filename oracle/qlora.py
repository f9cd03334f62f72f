"""QLoRA linear layer and QLoRA SwiGLU MLP: forward and hand-derived backward.

TEST INFRASTRUCTURE ONLY (see the package docstring): the plain CPU oracle.

Everything here is the plain definition evaluated in float64, with matrix
products as the only library primitive and no intermediate rounding.

Linear layer ("LLM Fine-Tuning in 2026: Unsloth vs QLoRA vs Liger-Kernel",
section 1, the LoRA update h = W0 x + (alpha/r) B A x; no dropout and no bias,
section 5's adapter settings).  With tokens as rows, X [M, K], frozen
dequantized W0 [N, K], A [r, K], B [N, r] and s = alpha / r:

    XA = X A^T                      [M, r]
    Y  = X W0^T + s XA B^T          [M, N]

Backward of the loss <Y, dY> (section 2 of the same page: gradients derived by
hand instead of by autograd; W0 is frozen, so it gets no gradient):

    T  = dY B                       [M, r]
    dX = dY W0 + s T A              [M, K]
    dB = s dY^T XA                  [N, r]
    dA = s T^T X                    [r, K]

Merge (the listing's 16-bit merge save step): W' = W0 + s B A in float64,
rounded once to bf16 or fp16 (nearest, ties to even).

SwiGLU MLP built from three such layers (gate, up: D -> I; down: I -> D;
"MLP SwiGLU" among the hand-derived kernels in section 2; the variant is
silu(gate) * up):

    G = lin_g(X), U = lin_u(X), H = silu(G) * U, Y = lin_d(H)
    silu(g) = g sigma(g),  silu'(g) = sigma(g) (1 + g (1 - sigma(g)))

The backward keeps only G and U from the forward and recomputes sigma, silu and
H from them ("What is Unsloth", "Recompute instead of store"):

    dH = dY Wd + s_d (dY Bd) Ad
    dU = dH * silu(G)
    dG = dH * U * silu'(G)
    dX = dG Wg + s_g (dG Bg) Ag + dU Wu + s_u (dU Bu) Au
    plus the LoRA gradients of the three layers as for the linear layer.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns as float64."""
    u = np.asarray(u16, np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def as_f64(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return x.astype(np.float64)


def lora_scale(alpha: float, r: int) -> float:
    return float(alpha) / float(r)


# ------------------------------------------------------------------ merge

def merge_weight(W, A, B, alpha):
    """W + (alpha/r) B A in float64: the update h = W0 x + (alpha/r) B A x of
    "LLM Fine-Tuning in 2026", section 1, folded into one weight, as the
    listing's 16-bit merge save step does after training."""
    W, A, B = as_f64(W), as_f64(A), as_f64(B)
    return W + lora_scale(alpha, A.shape[0]) * (B @ A)


def f64_to_bf16_bits(x) -> np.ndarray:
    """float64 -> bf16 bit patterns in one rounding, to nearest, ties to even
    (no intermediate fp32).  bf16 keeps 8 significant bits; below its smallest
    normal 2^-126 the spacing is 2^-133.  Finite values within bf16 range."""
    x = np.asarray(x, np.float64)
    _, e = np.frexp(x)                      # |x| in [2^(e-1), 2^e)
    q = np.maximum(e - 8, -133)             # exponent of the last kept bit
    y = np.ldexp(np.rint(np.ldexp(x, -q)), q)  # rint: nearest, ties to even
    return (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def f64_to_f16_bits(x) -> np.ndarray:
    """float64 -> fp16 bit patterns in one rounding, to nearest, ties to even
    (numpy's direct double -> half conversion)."""
    return np.asarray(x, np.float64).astype(np.float16).view(np.uint16)


def merge_16bit(W, A, B, alpha, dtype: str = "bf16") -> np.ndarray:
    """The merged weight rounded once to 16 bits ("bf16" or "f16"): uint16
    bit patterns [N, K]."""
    Wm = merge_weight(W, A, B, alpha)
    return f64_to_bf16_bits(Wm) if dtype == "bf16" else f64_to_f16_bits(Wm)


# ------------------------------------------------------------------ linear

def linear_forward(X, W, A, B, alpha):
    """Y = X W^T + (alpha/r) (X A^T) B^T; returns (Y, XA) in float64."""
    X, W, A, B = as_f64(X), as_f64(W), as_f64(A), as_f64(B)
    s = lora_scale(alpha, A.shape[0])
    XA = X @ A.T
    Y = X @ W.T + s * (XA @ B.T)
    return Y, XA


def linear_backward(dY, X, W, A, B, alpha):
    """Gradients of <Y, dY>: returns (dX, dA, dB) in float64."""
    dY, X, W, A, B = as_f64(dY), as_f64(X), as_f64(W), as_f64(A), as_f64(B)
    s = lora_scale(alpha, A.shape[0])
    XA = X @ A.T
    T = dY @ B
    dX = dY @ W + s * (T @ A)
    dB = s * (dY.T @ XA)
    dA = s * (T.T @ X)
    return dX, dA, dB


# ------------------------------------------------------------------ SwiGLU

def sigmoid(g):
    """1 / (1 + exp(-g)), evaluated without overflow for either sign."""
    g = np.asarray(g, np.float64)
    out = np.empty_like(g)
    pos = g >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-g[pos]))
    e = np.exp(g[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def silu(g):
    g = np.asarray(g, np.float64)
    return g * sigmoid(g)


def silu_grad(g):
    g = np.asarray(g, np.float64)
    sg = sigmoid(g)
    return sg * (1.0 + g * (1.0 - sg))


# ------------------------------------------------------------------ MLP

def mlp_forward(X, Wg, Wu, Wd, Ag, Bg, Au, Bu, Ad, Bd, alpha):
    """Returns dict(Y, G, U, H, XA_g, XA_u, HA_d), all float64."""
    G, XA_g = linear_forward(X, Wg, Ag, Bg, alpha)
    U, XA_u = linear_forward(X, Wu, Au, Bu, alpha)
    H = silu(G) * U
    Y, HA_d = linear_forward(H, Wd, Ad, Bd, alpha)
    return dict(Y=Y, G=G, U=U, H=H, XA_g=XA_g, XA_u=XA_u, HA_d=HA_d)


def mlp_backward(dY, X, G, U, Wg, Wu, Wd, Ag, Bg, Au, Bu, Ad, Bd, alpha):
    """Gradients of <Y, dY> given the saved G and U (H is recomputed).

    Returns dict(dX, dA_g, dB_g, dA_u, dB_u, dA_d, dB_d, dG, dU), float64.
    """
    G, U = as_f64(G), as_f64(U)
    H = silu(G) * U
    dH, dA_d, dB_d = linear_backward(dY, H, Wd, Ad, Bd, alpha)
    dU = dH * silu(G)
    dG = dH * U * silu_grad(G)
    dXg, dA_g, dB_g = linear_backward(dG, X, Wg, Ag, Bg, alpha)
    dXu, dA_u, dB_u = linear_backward(dU, X, Wu, Au, Bu, alpha)
    return dict(dX=dXg + dXu, dA_g=dA_g, dB_g=dB_g, dA_u=dA_u, dB_u=dB_u,
                dA_d=dA_d, dB_d=dB_d, dG=dG, dU=dU)


def mlp_forward_backward_rows(X, dY, Wg, Wu, Wd, Ag, Bg, Au, Bu, Ad, Bd, alpha,
                              chunk: int = 1024, keep=("Y", "dX")):
    """Whole-batch MLP forward + backward, processing tokens in row chunks.

    Every token row is independent except for the LoRA gradients, which are
    sums over rows; those are summed over the chunks.  ``keep`` names the
    per-row outputs to return in full (e.g. Y, dX, G, U).
    """
    M = np.asarray(X).shape[0]
    grads = {k: 0.0 for k in ("dA_g", "dB_g", "dA_u", "dB_u", "dA_d", "dB_d")}
    rows = {k: [] for k in keep}
    for m0 in range(0, M, chunk):
        m1 = min(M, m0 + chunk)
        f = mlp_forward(X[m0:m1], Wg, Wu, Wd, Ag, Bg, Au, Bu, Ad, Bd, alpha)
        b = mlp_backward(dY[m0:m1], X[m0:m1], f["G"], f["U"], Wg, Wu, Wd,
                         Ag, Bg, Au, Bu, Ad, Bd, alpha)
        for k in grads:
            grads[k] = grads[k] + b[k]
        for k in keep:
            rows[k].append(f[k] if k in f else b[k])
    out = {k: np.concatenate(v, axis=0) for k, v in rows.items()}
    out.update(grads)
    return out
