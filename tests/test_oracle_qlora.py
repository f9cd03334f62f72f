"""Pins of the oracle's QLoRA linear layer and SwiGLU MLP.

* forward: B = 0 (and alpha = 0) reduces to the plain base matmul, written as
  loops; the pages' per-token column-vector form h = W0 x + (alpha/r) B (A x);
  the merged-weight form X (W0 + s B A)^T; linearity in s;
* backward: central finite differences of L = <Y, dY> in every input the
  gradients are taken for (exact up to rounding for the linear layer, which is
  linear in each of X, A and B separately), B = 0 => dA == 0;
* SwiGLU: closed-form values of silu and its derivative, a finite-difference
  check of the derivative, and the B = 0 reduction of the whole block to the
  plain SwiGLU MLP written as loops.
"""
import math

import numpy as np
import pytest

import synth
from oracle import nf4, qlora


def _small_linear(M=3, K=64, N=5, r=2, seed=11, zero_B=False):
    rng = np.random.default_rng(seed)
    cb = synth.nf4_codebook()
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    Wh = nf4.dequantize(nf4.quantize(W, cb), cb).astype(np.float64)
    X = rng.standard_normal((M, K))
    A = rng.uniform(-0.2, 0.2, (r, K))
    B = np.zeros((N, r)) if zero_B else rng.standard_normal((N, r)) * 0.3
    dY = rng.standard_normal((M, N))
    return X, Wh, A, B, dY


def test_b_zero_is_plain_matmul():
    X, Wh, A, B, _ = _small_linear(zero_B=True)
    Y, _ = qlora.linear_forward(X, Wh, A, B, alpha=16.0)
    M, K = X.shape
    N = Wh.shape[0]
    for m in range(M):
        for n in range(N):
            ref = math.fsum(X[m, k] * Wh[n, k] for k in range(K))
            assert abs(Y[m, n] - ref) <= 1e-12 * (1 + abs(ref))


def test_alpha_zero_is_plain_matmul():
    X, Wh, A, B, _ = _small_linear()
    Y, _ = qlora.linear_forward(X, Wh, A, B, alpha=0.0)
    Y0, _ = qlora.linear_forward(X, Wh, A, np.zeros_like(B), alpha=16.0)
    assert np.array_equal(Y, Y0)


def test_column_vector_form_of_the_update():
    """h = W0 x + (alpha/r) B (A x) per token, evaluated with loops."""
    X, Wh, A, B, _ = _small_linear()
    alpha = 16.0
    r, K = A.shape
    N = Wh.shape[0]
    Y, XA = qlora.linear_forward(X, Wh, A, B, alpha)
    for m in range(X.shape[0]):
        x = X[m]
        Ax = [math.fsum(A[j, k] * x[k] for k in range(K)) for j in range(r)]
        for j in range(r):
            assert abs(XA[m, j] - Ax[j]) <= 1e-12 * (1 + abs(Ax[j]))
        for n in range(N):
            h = math.fsum(Wh[n, k] * x[k] for k in range(K)) + \
                (alpha / r) * math.fsum(B[n, j] * Ax[j] for j in range(r))
            assert abs(Y[m, n] - h) <= 1e-12 * (1 + abs(h))


def test_merged_weight_form_and_linearity_in_s():
    X, Wh, A, B, _ = _small_linear(r=3)
    Y1, _ = qlora.linear_forward(X, Wh, A, B, 3.0)   # s = 1
    Y2, _ = qlora.linear_forward(X, Wh, A, B, 6.0)   # s = 2
    Y0, _ = qlora.linear_forward(X, Wh, A, B, 0.0)
    np.testing.assert_allclose(Y2 - Y0, 2 * (Y1 - Y0), rtol=1e-12, atol=1e-12)
    merged = Wh + 2.0 * (B @ A)
    np.testing.assert_allclose(Y2, X @ merged.T, rtol=1e-12, atol=1e-12)


def _fd_grad(f, P, h):
    g = np.zeros_like(P)
    for idx in np.ndindex(P.shape):
        old = P[idx]
        P[idx] = old + h
        fp = f()
        P[idx] = old - h
        fm = f()
        P[idx] = old
        g[idx] = (fp - fm) / (2 * h)
    return g


def test_linear_backward_finite_differences():
    X, Wh, A, B, dY = _small_linear(M=3, K=64, N=64, r=2)
    alpha = 16.0

    def loss():
        return float(np.sum(qlora.linear_forward(X, Wh, A, B, alpha)[0] * dY))

    dX, dA, dB = qlora.linear_backward(dY, X, Wh, A, B, alpha)
    for P, G in ((X, dX), (A, dA), (B, dB)):
        g = _fd_grad(loss, P, 1e-3)
        np.testing.assert_allclose(G, g, rtol=1e-7, atol=1e-9)


def test_linear_b_zero_gives_zero_dA():
    X, Wh, A, B, dY = _small_linear(zero_B=True)
    _, dA, dB = qlora.linear_backward(dY, X, Wh, A, B, 16.0)
    assert np.all(dA == 0)
    assert np.any(dB != 0)


def test_silu_closed_forms():
    assert qlora.silu(np.array([0.0]))[0] == 0.0
    assert qlora.silu_grad(np.array([0.0]))[0] == 0.5
    x = np.linspace(-30, 30, 241)
    # silu(-x) = silu(x) - x
    np.testing.assert_allclose(qlora.silu(-x), qlora.silu(x) - x, rtol=1e-12, atol=1e-12)
    # saturation without overflow
    big = np.array([-800.0, 800.0])
    assert np.all(np.isfinite(qlora.sigmoid(big)))
    assert qlora.sigmoid(big)[0] == 0.0 and qlora.sigmoid(big)[1] == 1.0
    # sigma(1) from its definition
    assert abs(qlora.sigmoid(np.array([1.0]))[0] - 1 / (1 + math.exp(-1))) < 1e-15
    h = 1e-5
    xs = np.linspace(-8, 8, 33)
    fd = (qlora.silu(xs + h) - qlora.silu(xs - h)) / (2 * h)
    np.testing.assert_allclose(qlora.silu_grad(xs), fd, rtol=1e-8, atol=1e-9)


def _small_mlp(M=3, D=64, I=128, r=2, seed=21, zero_B=False):
    rng = np.random.default_rng(seed)
    cb = synth.nf4_codebook()

    def deq(n, k):
        W = (rng.standard_normal((n, k)) * 0.1).astype(np.float32)
        return nf4.dequantize(nf4.quantize(W, cb), cb).astype(np.float64)

    p = dict(Wg=deq(I, D), Wu=deq(I, D), Wd=deq(D, I),
             Ag=rng.uniform(-.2, .2, (r, D)), Au=rng.uniform(-.2, .2, (r, D)),
             Ad=rng.uniform(-.2, .2, (r, I)))
    for nm, n in (("Bg", I), ("Bu", I), ("Bd", D)):
        p[nm] = np.zeros((n, r)) if zero_B else rng.standard_normal((n, r)) * 0.3
    X = rng.standard_normal((M, D))
    dY = rng.standard_normal((M, D))
    return X, dY, p


def test_mlp_b_zero_is_plain_swiglu():
    X, _, p = _small_mlp(M=2, D=64, I=64, zero_B=True)
    Y = qlora.mlp_forward(X, p["Wg"], p["Wu"], p["Wd"], p["Ag"], p["Bg"], p["Au"], p["Bu"],
                          p["Ad"], p["Bd"], 16.0)["Y"]
    D, I = 64, 64
    for m in range(2):
        h = []
        for i in range(I):
            g = math.fsum(X[m, k] * p["Wg"][i, k] for k in range(D))
            u = math.fsum(X[m, k] * p["Wu"][i, k] for k in range(D))
            h.append(g / (1 + math.exp(-g)) * u)
        for d in range(D):
            ref = math.fsum(h[i] * p["Wd"][d, i] for i in range(I))
            assert abs(Y[m, d] - ref) <= 1e-11 * (1 + abs(ref))


def test_mlp_backward_finite_differences():
    X, dY, p = _small_mlp()
    alpha = 8.0
    names = ("Wg", "Wu", "Wd", "Ag", "Bg", "Au", "Bu", "Ad", "Bd")

    def fwd():
        return qlora.mlp_forward(X, *[p[k] for k in names], alpha)

    def loss():
        return float(np.sum(fwd()["Y"] * dY))

    f = fwd()
    g = qlora.mlp_backward(dY, X, f["G"], f["U"], *[p[k] for k in names], alpha)
    checks = [(X, g["dX"])] + [(p[k], g["d%s_%s" % (k[0], k[1])])
                               for k in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd")]
    for P, G in checks:
        fd = _fd_grad(loss, P, 1e-5)
        np.testing.assert_allclose(G, fd, rtol=2e-6, atol=1e-7)


def test_mlp_row_chunks_equal_whole():
    X, dY, p = _small_mlp(M=7)
    names = ("Wg", "Wu", "Wd", "Ag", "Bg", "Au", "Bu", "Ad", "Bd")
    W = [p[k] for k in names]
    f = qlora.mlp_forward(X, *W, 16.0)
    b = qlora.mlp_backward(dY, X, f["G"], f["U"], *W, 16.0)
    c = qlora.mlp_forward_backward_rows(X, dY, *W, 16.0, chunk=3, keep=("Y", "dX", "G"))
    np.testing.assert_allclose(c["Y"], f["Y"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(c["G"], f["G"], rtol=1e-13, atol=1e-13)
    for k in ("dX", "dA_g", "dB_g", "dA_u", "dB_u", "dA_d", "dB_d"):
        np.testing.assert_allclose(c[k], b[k], rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ merge

def test_merge_weight_is_the_forward_weight():
    """The merged weight reproduces the layer's forward (linear_forward is a
    separate function): a wrong scale or a transposed B A fails here."""
    X, Wh, A, B, _ = _small_linear(M=4, K=64, N=7, r=3)
    for alpha in (3.0, 16.0):
        Y, _ = qlora.linear_forward(X, Wh, A, B, alpha)
        np.testing.assert_allclose(X @ qlora.merge_weight(Wh, A, B, alpha).T, Y, rtol=1e-12, atol=1e-12)


def test_merge_b_zero_is_dequantize_bits():
    rng = np.random.default_rng(5)
    cb = synth.nf4_codebook()
    W = (rng.standard_normal((8, 128)) * 0.02).astype(np.float32)
    for dq in (0, 256):
        qw = nf4.quantize(W, cb, dq_group=dq)
        Wh = nf4.dequantize(qw, cb)
        A = rng.uniform(-0.1, 0.1, (4, 128))
        got = qlora.merge_16bit(Wh, A, np.zeros((8, 4)), 16.0, "bf16")
        assert np.array_equal(got, nf4.dequantize_bf16(qw, cb))


def _bits_to_f64(bits, dtype):
    bits = np.asarray(bits, np.uint16)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


def _check_nearest_even(x, bits, dtype):
    """Brute force: the rounded value is at least as close to x as both 16-bit
    neighbours, and on an exact tie its last mantissa bit is 0."""
    y = _bits_to_f64(bits, dtype)
    for step in (-1, 1):
        nb = (bits.astype(np.int32) + step * np.where(y >= 0, 1, -1)).astype(np.uint16)
        z = _bits_to_f64(nb, dtype)
        dy, dz = np.abs(y - x), np.abs(z - x)
        assert np.all(dy <= dz), (x[dy > dz][:5], y[dy > dz][:5])
        tie = dy == dz
        assert np.all((bits[tie] & 1) == 0)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_one_step_16bit_rounding(dtype):
    rng = np.random.default_rng(9)
    conv = qlora.f64_to_bf16_bits if dtype == "bf16" else qlora.f64_to_f16_bits
    # random values of several magnitudes
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-12, 12, 20000))
    _check_nearest_even(x, conv(x), dtype)
    # exact ties between neighbours, and values a hair above a tie (below fp32
    # resolution there, so a rounding through fp32 would treat them as ties)
    b = conv(rng.standard_normal(4000))
    lo = _bits_to_f64(b, dtype)
    hi = _bits_to_f64((b.astype(np.int32) + np.where(lo >= 0, 1, -1)).astype(np.uint16), dtype)
    tie = (lo + hi) / 2
    _check_nearest_even(tie, conv(tie), dtype)
    above = tie + (hi - lo) * 2.0 ** -40
    got = conv(above)
    assert np.array_equal(_bits_to_f64(got, dtype), hi)
