"""The seeded input generator matches its published definition.

SplitMix64 output function (Steele, Lea & Flood, OOPSLA 2014) in counter mode
and Box-Muller, re-evaluated here with Python integers and floats.
"""
import math

import numpy as np

import synth

M64 = (1 << 64) - 1
G = 0x9E3779B97F4A7C15


def mix(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def py_bits(seed, stream, i):
    key = mix((seed * G + stream) & M64)
    return mix((key + (i + 1) * G) & M64)


def test_bits_match_definition():
    for seed, stream in ((0, 0), (1000, 2), (2 ** 40 + 7, 11)):
        for i in (0, 1, 2, 1000, 2 ** 33):
            assert synth.bits(seed, stream, i) == py_bits(seed, stream, i)


def test_normal_and_uniform_match_definition():
    seed, stream = 1003, 5
    z = synth.normal_f32(seed, stream, 50, 0.0, 0.02, offset=17)
    u = synth.uniform_f32(seed, stream, 50, -0.5, 0.25, offset=3)
    for i in range(50):
        u1 = 1.0 - (py_bits(seed, stream, 2 * (17 + i)) >> 11) * 2.0 ** -53
        u2 = (py_bits(seed, stream, 2 * (17 + i) + 1) >> 11) * 2.0 ** -53
        ref = 0.02 * (math.sqrt(-2 * math.log(u1)) * math.cos(2 * math.pi * u2))
        assert abs(float(z[i]) - ref) <= 1e-7 * max(1e-3, abs(ref))
        uu = (py_bits(seed, stream, 3 + i) >> 11) * 2.0 ** -53
        assert abs(float(u[i]) - (-0.5 + 0.75 * uu)) <= 1e-7


def test_bf16_is_rne_of_fp32():
    import torch
    f = synth.normal_f32(1, 1, 4096)
    b = synth.normal_bf16(1, 1, 4096)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


def test_moments_and_offsets():
    z = synth.normal_f32(7, 1, 1 << 20)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    tail = synth.normal_f32(7, 1, 100, offset=(1 << 20) - 100)
    assert np.array_equal(tail, z[-100:])
    rows = synth.weight_rows(5, 2, 128, 3, 2)
    full = synth.normal_f32(5, 2, 5 * 128, 0.0, synth.W_STD).reshape(5, 128)
    assert np.array_equal(rows, full[3:5])
