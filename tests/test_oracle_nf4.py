"""Pins of the oracle's NF4 quantizer / dequantizer against what the format fixes.

Every check here is independent of the oracle's own code path: exact rational
brute force for the nearest-code search, hand-built blocks whose codes are
known, round trips, and error bounds that follow from the definitions.
"""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import nf4

DYADIC = np.array([-1, -0.75, -0.5, -0.375, -0.25, -0.125, -0.0625, 0,
                   0.0625, 0.125, 0.25, 0.375, 0.5, 0.625, 0.75, 1], np.float32)


def brute_code(w: np.float32, a: np.float32, cb: np.ndarray) -> int:
    """Nearest codebook entry to fp32(w / a), ties to the lower index, exactly."""
    if a == 0:
        return int(np.flatnonzero(cb == 0)[0])
    # fp64 rounding of the exact quotient, then fp32: innocuous double rounding
    # for division (53 >= 2*24 + 2), so this is the correctly rounded fp32 quotient.
    n = np.float32(float(Fraction(float(w)) / Fraction(float(a))))
    dist = [abs(Fraction(float(n)) - Fraction(float(c))) for c in cb]
    best = min(dist)
    return dist.index(best)


def test_codebook_shape(codebook):
    cb = codebook
    assert cb.dtype == np.float32 and cb.shape == (16,)
    assert np.all(np.diff(cb.astype(np.float64)) > 0)
    assert cb[0] == -1.0 and cb[15] == 1.0 and cb[7] == 0.0
    assert np.count_nonzero(cb == 0) == 1


def test_codebook_golden(codebook):
    """The stored table (tests/golden/nf4_codebook.txt) matches the generator."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "nf4_codebook.txt")
    vals = [float.fromhex(line.split()[0]) for line in open(path)
            if line.strip() and not line.startswith("#")]
    assert np.array_equal(np.array(vals, np.float32), codebook)


def test_midpoints_exact(codebook):
    m = nf4.midpoints(codebook)
    for j in range(15):
        assert Fraction(m[j]) == (Fraction(float(codebook[j])) + Fraction(float(codebook[j + 1]))) / 2


@pytest.mark.parametrize("cbname", ["normal", "dyadic"])
def test_codes_brute_force_random(codebook, cbname):
    cb = codebook if cbname == "normal" else DYADIC
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((4, 128)) * 0.02).astype(np.float32)
    W[1, :64] *= 1e-3
    W[2, 64:] = 0.0
    q = nf4.unpack_nibbles(nf4.quantize(W, cb)["codes"], W.size).reshape(W.shape)
    a = nf4.absmax_blocks(W).reshape(4, 2)
    for i in range(4):
        for k in range(128):
            assert q[i, k] == brute_code(W[i, k], a[i, k // 64], cb), (i, k)


def test_codes_near_every_midpoint(codebook):
    """Values just below, at and above every midpoint (block absmax = 1)."""
    cb = codebook
    vals = [1.0]
    for m in nf4.midpoints(cb):
        f = np.float32(m)
        vals += [f, np.nextafter(f, np.float32(-2)), np.nextafter(f, np.float32(2))]
    vals = np.array(vals, np.float32)
    W = np.zeros((1, 64 * ((vals.size + 63) // 64)), np.float32)
    W[0, :vals.size] = vals
    q = nf4.unpack_nibbles(nf4.quantize(W, cb)["codes"], W.size)
    a = nf4.absmax_blocks(W)
    for k in range(vals.size):
        assert q[k] == brute_code(W[0, k], a[k // 64], cb), k


def test_ties_go_to_lower_index():
    cb = DYADIC
    W = np.zeros((1, 64), np.float32)
    W[0, 0] = 1.0                                    # absmax 1
    W[0, 1] = 0.03125                                # midpoint of 0 and 0.0625
    W[0, 2] = -0.03125                               # midpoint of -0.0625 and 0
    W[0, 3] = 0.875                                  # midpoint of 0.75 and 1
    W[0, 4] = -0.875                                 # midpoint of -1 and -0.75
    q = nf4.unpack_nibbles(nf4.quantize(W, cb)["codes"], 64)
    assert list(q[:5]) == [15, 7, 6, 14, 0]


def test_nibble_order_and_codebook_exact_block(codebook):
    """A block holding codebook entries * 2^e encodes to exactly those indices."""
    cb = codebook
    idx = np.array([(5 * i + 3) % 16 for i in range(64)])
    idx[10] = 15  # make sure +1 (the absmax) is present
    for e in (-7, 0, 3):
        W = (cb[idx] * np.float32(2.0 ** e)).astype(np.float32).reshape(1, 64)
        qw = nf4.quantize(W, cb)
        assert qw["absmax"][0] == np.float32(2.0 ** e)
        c = qw["codes"]
        assert c[0] == (idx[0] | (idx[1] << 4))
        assert c[1] == (idx[2] | (idx[3] << 4))
        assert np.array_equal(nf4.unpack_nibbles(c, 64), idx.astype(np.uint8))
        assert np.array_equal(nf4.dequantize(qw, cb), W)


def test_block_max_maps_to_extreme(codebook):
    rng = np.random.default_rng(1)
    W = rng.standard_normal((8, 256)).astype(np.float32)
    qw = nf4.quantize(W, codebook)
    q = nf4.unpack_nibbles(qw["codes"], W.size).reshape(-1, 64)
    blocks = W.reshape(-1, 64)
    am = np.argmax(np.abs(blocks), axis=1)
    for b in range(blocks.shape[0]):
        assert q[b, am[b]] == (15 if blocks[b, am[b]] > 0 else 0)


def test_zero_negzero_subnormal_blocks(codebook):
    cb = codebook
    z = 7
    W = np.zeros((1, 256), np.float32)
    W[0, 64:128] = -0.0                                       # all -0.0 block
    W[0, 128:192] = np.float32(1e-40) * np.linspace(-1, 1, 64).astype(np.float32)
    W[0, 192] = 0.5
    W[0, 193] = -0.0
    qw = nf4.quantize(W, cb)
    q = nf4.unpack_nibbles(qw["codes"], 256)
    assert np.all(q[:128] == z)
    assert qw["absmax"][0] == 0 and qw["absmax"][1] == 0
    assert qw["absmax"][2] > 0 and qw["absmax"][2] < np.finfo(np.float32).tiny
    for k in range(128, 256):
        assert q[k] == brute_code(W[0, k], qw["absmax"][k // 64], cb), k
    assert q[193] == z
    assert np.all(nf4.dequantize(qw, cb)[0, :128] == 0)


@pytest.mark.parametrize("dq", [0, 256])
def test_idempotence(codebook, dq):
    cb = codebook
    W = synth.weight_rows(1234, 2, 512, 0, 40)
    q1 = nf4.quantize(W, cb, dq_group=dq)
    W1 = nf4.dequantize(q1, cb)
    q2 = nf4.quantize(W1, cb, dq_group=dq)
    assert np.array_equal(q1["codes"], q2["codes"])
    if dq:
        assert np.array_equal(q1["absmax_q"], q2["absmax_q"])
        s1, s2 = q1["absmax_scale"], q2["absmax_scale"]
        assert np.all(np.abs(s1 - s2) <= np.spacing(s1))
    else:
        assert np.array_equal(q1["absmax"], q2["absmax"])
        assert np.array_equal(nf4.dequantize(q2, cb), W1)


def test_dequant_error_bound(codebook):
    cb = codebook
    W = synth.weight_rows(99, 2, 1024, 0, 16)
    qw = nf4.quantize(W, cb)
    Wh = nf4.dequantize(qw, cb)
    a = np.repeat(qw["absmax"], 64).reshape(W.shape).astype(np.float64)
    gap = np.max(np.diff(cb.astype(np.float64)))
    err = np.abs(W.astype(np.float64) - Wh.astype(np.float64))
    assert np.all(err <= a * (gap / 2 + 2.0 ** -23) + np.spacing(np.float32(a.max())))


def test_double_quant_properties():
    rng = np.random.default_rng(3)
    a = np.abs(rng.standard_normal(1000)).astype(np.float32)
    a[300:556] = 0.0                                  # an all-zero group (blocks 256..511 partly)
    a[256:512] = 0.0
    codes8, S = nf4.double_quantize(a, 256)
    assert S.shape == (4,)
    assert S[1] == 0 and np.all(codes8[256:512] == 0)
    for g in range(4):
        seg = a[g * 256:(g + 1) * 256]
        if seg.max() == 0:
            continue
        assert S[g] == np.float32(float(Fraction(float(seg.max())) / 255))
        assert codes8[g * 256 + int(np.argmax(seg))] == 255
    ah = nf4.dq_absmax(codes8, S, 256)
    Sg = np.repeat(S, 256)[:1000].astype(np.float64)
    assert np.all(np.abs(ah - a.astype(np.float64)) <= Sg / 2 + np.spacing(a))


def test_dq_codes_round_half_even():
    # S = 1/255 * 255 / 255 ... construct a group with max 255 so S == 1 exactly
    a = np.array([255.0, 2.5, 3.5, 0.5, 1.5, 254.5], np.float32)
    codes8, S = nf4.double_quantize(a, 256)
    assert S[0] == 1.0
    assert list(codes8) == [255, 2, 4, 0, 2, 254]


def test_bf16_export_matches_torch_rne(codebook):
    torch = pytest.importorskip("torch")
    W = synth.weight_rows(7, 2, 256, 0, 32)
    qw = nf4.quantize(W, codebook)
    f = nf4.dequantize(qw, codebook)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(nf4.dequantize_bf16(qw, codebook), ref)
    # and exact halfway cases of the rounding itself
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)], np.float32)
    refx = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(nf4.to_bf16_bits(x), refx)
