"""Seeded synthetic inputs for the QLoRA linear / SwiGLU-MLP workloads.

This module is shared by the CPU oracle and the GPU path.  It holds no
arithmetic of the method itself: only the random-number recipe (``synth.c``),
the fixed NF4 codebook table that both sides receive as an input, and the
shapes of the five workloads.

Workload shapes and distributions follow the QLoRA fine-tuning setup the
pages describe (frozen 4-bit NF4 base weight, LoRA rank r, scale alpha/r,
"LLM Fine-Tuning in 2026: Unsloth vs QLoRA vs Liger-Kernel", section 1 and
section 5; batch 2 x sequence 2048 tokens, section 5): Llama-3-8B and
Llama-3-70B projection shapes.  Values are synthetic; no dataset or trained
weight is used.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile ``synth.c`` with gcc + OpenMP into ``libsynth.so`` (in-tree)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11",
                               os.path.join(_HERE, "synth.c"), "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i64, d = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double
        vp = ctypes.c_void_p
        lib.synth_bits.restype = u64
        lib.synth_bits.argtypes = [u64, u64, u64]
        for name in ("synth_normal_f32", "synth_normal_bf16", "synth_uniform_f32",
                     "synth_uniform_bf16"):
            f = getattr(lib, name)
            f.restype = None
            f.argtypes = [u64, u64, i64, u64, d, d, vp]
        _lib = lib
    return _lib


# ---------------------------------------------------------------- generators

def bits(seed: int, stream: int, i: int) -> int:
    return int(_load().synth_bits(seed, stream, i))


def normal_f32(seed, stream, n, mean=0.0, std=1.0, offset=0):
    out = np.empty(int(n), np.float32)
    _load().synth_normal_f32(seed, stream, int(n), offset, mean, std, out.ctypes.data)
    return out


def normal_bf16(seed, stream, n, mean=0.0, std=1.0, offset=0):
    """bf16 bit patterns (uint16), fp64 value -> fp32 (RN) -> bf16 (RNE)."""
    out = np.empty(int(n), np.uint16)
    _load().synth_normal_bf16(seed, stream, int(n), offset, mean, std, out.ctypes.data)
    return out


def uniform_f32(seed, stream, n, lo, hi, offset=0):
    out = np.empty(int(n), np.float32)
    _load().synth_uniform_f32(seed, stream, int(n), offset, lo, hi, out.ctypes.data)
    return out


def uniform_bf16(seed, stream, n, lo, hi, offset=0):
    out = np.empty(int(n), np.uint16)
    _load().synth_uniform_bf16(seed, stream, int(n), offset, lo, hi, out.ctypes.data)
    return out


def targets(seed, stream, n, V, ignore_every=0, ignore_index=-100):
    """n class indices in [0, V) from the counter-based bits (bits mod V);
    with ignore_every = k > 0, every k-th index (i % k == k - 1) is the
    ignore value instead."""
    out = np.empty(int(n), np.int32)
    for i in range(int(n)):
        out[i] = ignore_index if ignore_every and i % ignore_every == ignore_every - 1 else bits(seed, stream, i) % V
    return out


def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(u16, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ------------------------------------------------------------ NF4 codebook

P_MAX = 0.97  # outermost normal-quantile probability used for the table


def _norm_ppf(p: float) -> float:
    """Inverse standard normal CDF by bisection on Phi(x) = erfc(-x/sqrt2)/2."""
    lo, hi = -12.0, 12.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if 0.5 * math.erfc(-mid / math.sqrt(2.0)) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def nf4_codebook() -> np.ndarray:
    """The fixed 16-entry normal-quantile codebook given to both sides.

    A 4-bit NormalFloat table (the QLoRA weight format named on the pages,
    "LLM Fine-Tuning in 2026", FAQ on LoRA vs QLoRA): 8 positive levels at
    equally spaced probabilities in (1/2, P_MAX], 7 negative levels likewise,
    each half scaled so that its extreme is exactly +-1, plus an exact 0.
    Strictly increasing fp32, c[0] = -1, c[7] = 0, c[15] = +1.
    """
    pos = [_norm_ppf(0.5 + i * (P_MAX - 0.5) / 8) for i in range(1, 9)]
    neg = [_norm_ppf(0.5 + i * (P_MAX - 0.5) / 7) for i in range(1, 8)]
    vals = [-v / neg[-1] for v in reversed(neg)] + [0.0] + [v / pos[-1] for v in pos]
    cb = np.array(vals, np.float64).astype(np.float32)
    cb[0], cb[7], cb[15] = -1.0, 0.0, 1.0
    return cb


# ------------------------------------------------------------ workloads

@dataclass(frozen=True)
class LinearCfg:
    name: str
    M: int
    K: int  # in features
    N: int  # out features
    r: int
    alpha: float
    dq_group: int  # 0 = fp32 absmax, 256 = double-quantized absmax
    blocksize: int = 64
    kind: str = "linear"


@dataclass(frozen=True)
class MlpCfg:
    name: str
    M: int
    D: int  # hidden
    I: int  # intermediate
    r: int
    alpha: float
    dq_group: int
    blocksize: int = 64
    kind: str = "mlp"


CONFIGS = [
    LinearCfg("linear_m256_512x512_r8", M=256, K=512, N=512, r=8, alpha=16.0, dq_group=0),
    LinearCfg("llama3_8b_q_proj_m4096_r16", M=4096, K=4096, N=4096, r=16, alpha=16.0, dq_group=0),
    MlpCfg("llama3_8b_mlp_m8192_r16", M=8192, D=4096, I=14336, r=16, alpha=16.0, dq_group=0),
    MlpCfg("llama3_70b_mlp_m4096_r64_dq", M=4096, D=8192, I=28672, r=64, alpha=16.0, dq_group=256),
    LinearCfg("skinny_gate_proj_m64_8192x28672_r16_dq", M=64, K=8192, N=28672, r=16, alpha=16.0,
              dq_group=256),
]


def seed_of(index: int) -> int:
    return 1000 + index


W_STD = 0.02
B_STD = 0.01

# stream ids of each tensor
LIN_STREAMS = dict(X=1, W0=2, A=3, B=4, dY=5)
MLP_STREAMS = dict(X=1, Wg=2, Wu=3, Wd=4, Ag=5, Bg=6, Au=7, Bu=8, Ad=9, Bd=10, dY=11)


def linear_inputs(cfg: LinearCfg, seed: int, M: int | None = None, with_weight: bool = True):
    """Inputs of one QLoRA linear: X, W0 (fp32), A, B, dY (bf16 as uint16).

    X ~ N(0,1), W0 ~ N(0, 0.02), A ~ U(-1/sqrt(in), 1/sqrt(in)), B ~ N(0, 0.01),
    dY ~ N(0,1).  ``M`` may select the first rows of X / dY (row i of X is the
    same whatever M is).
    """
    M = cfg.M if M is None else M
    s = LIN_STREAMS
    bound = 1.0 / math.sqrt(cfg.K)
    out = dict(
        X=normal_bf16(seed, s["X"], M * cfg.K).reshape(M, cfg.K),
        A=uniform_bf16(seed, s["A"], cfg.r * cfg.K, -bound, bound).reshape(cfg.r, cfg.K),
        B=normal_bf16(seed, s["B"], cfg.N * cfg.r, 0.0, B_STD).reshape(cfg.N, cfg.r),
        dY=normal_bf16(seed, s["dY"], M * cfg.N).reshape(M, cfg.N),
    )
    if with_weight:
        out["W0"] = normal_f32(seed, s["W0"], cfg.N * cfg.K, 0.0, W_STD).reshape(cfg.N, cfg.K)
    return out


def weight_rows(seed: int, stream: int, K: int, row0: int, nrows: int) -> np.ndarray:
    """Rows [row0, row0+nrows) of an fp32 N(0, 0.02) weight of row length K."""
    return normal_f32(seed, stream, nrows * K, 0.0, W_STD, offset=row0 * K).reshape(nrows, K)


def mlp_inputs(cfg: MlpCfg, seed: int, M: int | None = None, with_weights: bool = True):
    """Inputs of one QLoRA SwiGLU MLP (gate/up: D->I, down: I->D)."""
    M = cfg.M if M is None else M
    s = MLP_STREAMS
    D, I, r = cfg.D, cfg.I, cfg.r
    bD, bI = 1.0 / math.sqrt(D), 1.0 / math.sqrt(I)
    out = dict(
        X=normal_bf16(seed, s["X"], M * D).reshape(M, D),
        Ag=uniform_bf16(seed, s["Ag"], r * D, -bD, bD).reshape(r, D),
        Bg=normal_bf16(seed, s["Bg"], I * r, 0.0, B_STD).reshape(I, r),
        Au=uniform_bf16(seed, s["Au"], r * D, -bD, bD).reshape(r, D),
        Bu=normal_bf16(seed, s["Bu"], I * r, 0.0, B_STD).reshape(I, r),
        Ad=uniform_bf16(seed, s["Ad"], r * I, -bI, bI).reshape(r, I),
        Bd=normal_bf16(seed, s["Bd"], D * r, 0.0, B_STD).reshape(D, r),
        dY=normal_bf16(seed, s["dY"], M * D).reshape(M, D),
    )
    if with_weights:
        out["Wg"] = normal_f32(seed, s["Wg"], I * D, 0.0, W_STD).reshape(I, D)
        out["Wu"] = normal_f32(seed, s["Wu"], I * D, 0.0, W_STD).reshape(I, D)
        out["Wd"] = normal_f32(seed, s["Wd"], D * I, 0.0, W_STD).reshape(D, I)
    return out
