"""Thin Python binding of libqlora.so (include/qlora.h) for MI355X / gfx950.

Argument marshalling only: torch supplies device memory (``torch.empty``) and
the current HIP stream; every step of the computation runs in the library's
HIP kernels.  Each function carries the name of the C entry point it calls.
If the compiled library is missing, importing the ABI raises immediately:
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora.so")

QLORA_OK = 0
QLORA_DTYPE_BF16 = 0
QLORA_DTYPE_F32 = 1
QLORA_DTYPE_F16 = 2

EXPORTED = (
    "qlora_abi_version", "qlora_strerror", "nf4_quantize", "nf4_dequantize",
    "qlora_linear_workspace_bytes", "qlora_linear_fwd", "qlora_linear_bwd",
    "qlora_mlp_workspace_bytes", "qlora_mlp_fwd", "qlora_mlp_bwd", "qlora_trace_install", "qlora_merge",
    "rmsnorm_fwd", "rmsnorm_bwd", "rmsnorm_bwd_workspace_bytes",
    "qlora_grouped_workspace_bytes", "qlora_grouped_fwd", "qlora_grouped_bwd",
    "qlora_linear_ce_workspace_bytes", "qlora_linear_ce", "qlora_linear_fwd_static", "qlora_debug_force_arch",
    "qlora_mlp_rmsnorm_workspace_bytes", "qlora_mlp_fwd_rmsnorm",
)
QLORA_STATIC_SCRATCH_BYTES = 64 << 20


class QloraError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__("%s failed: %d (%s)" % (fn, status, msg))
        self.status = status


# ------------------------------------------------------------------ C structs

class CNf4(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("absmax", ctypes.c_void_p),
                ("absmax_q", ctypes.c_void_p), ("absmax_scale", ctypes.c_void_p),
                ("codebook", ctypes.c_void_p), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("blocksize", ctypes.c_int32), ("dq_group", ctypes.c_int32)]


class CLinear(ctypes.Structure):
    _fields_ = [("W0", CNf4), ("A", ctypes.c_void_p), ("B", ctypes.c_void_p),
                ("r", ctypes.c_int32), ("alpha", ctypes.c_float)]


class CGrouped(ctypes.Structure):
    _fields_ = [("W0", CNf4), ("A", ctypes.c_void_p), ("B", ctypes.c_void_p * 8), ("N", ctypes.c_int32 * 8),
                ("r", ctypes.c_int32 * 8), ("alpha", ctypes.c_float * 8), ("G", ctypes.c_int32)]


class CMlp(ctypes.Structure):
    _fields_ = [("gate", CLinear), ("up", CLinear), ("down", CLinear)]


class CMlpSaved(ctypes.Structure):
    _fields_ = [("G", ctypes.c_void_p), ("U", ctypes.c_void_p), ("XA_g", ctypes.c_void_p),
                ("XA_u", ctypes.c_void_p), ("HA_d", ctypes.c_void_p)]


class CMlpGrads(ctypes.Structure):
    _fields_ = [("dA_g", ctypes.c_void_p), ("dB_g", ctypes.c_void_p), ("dA_u", ctypes.c_void_p),
                ("dB_u", ctypes.c_void_p), ("dA_d", ctypes.c_void_p), ("dB_d", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libqlora.so and declare its signatures (no GPU needed)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libqlora.so not built (%s); run `python -m qlora_fine_tuning_linear_amd.build`"
                           % path)
    lib = ctypes.CDLL(path)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    P = ctypes.POINTER
    sig = {
        "qlora_abi_version": (ctypes.c_uint32, []),
        "qlora_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "nf4_quantize": (ctypes.c_int, [vp, i64, i64, vp, i32, i32, vp, vp, vp, vp, vp]),
        "nf4_dequantize": (ctypes.c_int, [P(CNf4), i32, vp, vp]),
        "qlora_linear_workspace_bytes": (sz, [P(CLinear), i64]),
        "qlora_linear_fwd": (ctypes.c_int, [P(CLinear), vp, i64, vp, vp, vp, sz, vp]),
        "qlora_linear_bwd": (ctypes.c_int, [P(CLinear), vp, vp, vp, i64, vp, vp, vp, vp, sz, vp]),
        "qlora_mlp_workspace_bytes": (sz, [P(CMlp), i64]),
        "qlora_mlp_fwd": (ctypes.c_int, [P(CMlp), vp, i64, vp, P(CMlpSaved), vp, sz, vp]),
        "qlora_mlp_rmsnorm_workspace_bytes": (sz, [P(CMlp), i64]),
        "qlora_mlp_fwd_rmsnorm": (ctypes.c_int, [P(CMlp), vp, vp, ctypes.c_float, i64, vp, P(CMlpSaved), vp, vp,
                                                 vp, sz, vp]),
        "qlora_mlp_bwd": (ctypes.c_int, [P(CMlp), vp, vp, P(CMlpSaved), i64, vp, P(CMlpGrads), vp, sz,
                                         vp]),
        "qlora_trace_install": (ctypes.c_int, [P(vp), P(vp), P(i32), i32, P(i32)]),
        "qlora_merge": (ctypes.c_int, [P(CLinear), i32, vp, vp]),
        "rmsnorm_fwd": (ctypes.c_int, [vp, vp, i64, i64, ctypes.c_float, vp, vp, vp]),
        "rmsnorm_bwd": (ctypes.c_int, [vp, vp, vp, vp, i64, i64, vp, vp, vp, sz, vp]),
        "rmsnorm_bwd_workspace_bytes": (sz, [i64, i64]),
        "qlora_grouped_workspace_bytes": (sz, [P(CGrouped), i64]),
        "qlora_grouped_fwd": (ctypes.c_int, [P(CGrouped), vp, i64, vp, vp, vp, sz, vp]),
        "qlora_grouped_bwd": (ctypes.c_int, [P(CGrouped), vp, vp, vp, i64, vp, vp, P(vp), vp, sz, vp]),
        "qlora_linear_ce_workspace_bytes": (sz, [i64, i64, i64, i64, i32]),
        "qlora_linear_ce": (ctypes.c_int, [vp, i64, i64, vp, i64, vp, i32, i64, vp, vp, vp, vp, sz, vp]),
        "qlora_linear_fwd_static": (ctypes.c_int, [P(CLinear), vp, i64, vp, vp, vp]),
        "qlora_debug_force_arch": (ctypes.c_int, [ctypes.c_char_p]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, st: int):
    if st != QLORA_OK:
        raise QloraError(fn, st, load_library().qlora_strerror(st).decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, dtype, shape, name):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError("%s: expected contiguous %s %s, got %s %s" % (name, dtype, tuple(shape), t.dtype,
                                                                     tuple(t.shape)))


# ------------------------------------------------------------------ NF4 weight

@dataclass
class Nf4Weight:
    codes: torch.Tensor                 # uint8 [N*K/2]
    absmax: Optional[torch.Tensor]      # fp32 [N*K/64]         (dq_group == 0)
    absmax_q: Optional[torch.Tensor]    # uint8 [N*K/64]        (dq_group == 256)
    absmax_scale: Optional[torch.Tensor]  # fp32 [ceil(nb/256)] (dq_group == 256)
    codebook: torch.Tensor              # fp32 [16]
    N: int
    K: int
    dq_group: int = 0
    blocksize: int = 64

    def c(self) -> CNf4:
        return CNf4(_ptr(self.codes), _ptr(self.absmax), _ptr(self.absmax_q), _ptr(self.absmax_scale),
                    _ptr(self.codebook), self.N, self.K, self.blocksize, self.dq_group)


def nf4_quantize(W: torch.Tensor, codebook: torch.Tensor, dq_group: int = 0, blocksize: int = 64) -> Nf4Weight:
    """nf4_quantize: fp32 [N, K] device weight -> NF4 codes + absmax (or DQ absmax)."""
    lib = load_library()
    N, K = W.shape
    _need(W, torch.float32, (N, K), "W")
    _need(codebook, torch.float32, (16,), "codebook")
    dev = W.device
    nb = N * K // blocksize
    codes = torch.empty(N * K // 2, dtype=torch.uint8, device=dev)
    absmax = absmax_q = scale = None
    if dq_group:
        absmax_q = torch.empty(nb, dtype=torch.uint8, device=dev)
        scale = torch.empty(-(-nb // dq_group), dtype=torch.float32, device=dev)
    else:
        absmax = torch.empty(nb, dtype=torch.float32, device=dev)
    st = lib.nf4_quantize(W.data_ptr(), N, K, codebook.data_ptr(), blocksize, dq_group, codes.data_ptr(),
                          _ptr(absmax), _ptr(absmax_q), _ptr(scale), _stream(dev))
    _check("nf4_quantize", st)
    return Nf4Weight(codes, absmax, absmax_q, scale, codebook, N, K, dq_group, blocksize)


def nf4_dequantize(w: Nf4Weight, dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None):
    """nf4_dequantize: NF4 weight -> bf16 or fp32 [N, K]."""
    lib = load_library()
    if out is None:
        out = torch.empty(w.N, w.K, dtype=dtype, device=w.codes.device)
    code = QLORA_DTYPE_F32 if out.dtype == torch.float32 else QLORA_DTYPE_BF16
    cw = w.c()
    _check("nf4_dequantize", lib.nf4_dequantize(ctypes.byref(cw), code, out.data_ptr(), _stream(out.device)))
    return out


# ------------------------------------------------------------------ linear

@dataclass
class QLoraLinear:
    W0: Nf4Weight
    A: torch.Tensor   # bf16 [r, K]
    B: torch.Tensor   # bf16 [N, r]
    alpha: float

    @property
    def r(self) -> int:
        return int(self.A.shape[0])

    def c(self) -> CLinear:
        return CLinear(self.W0.c(), self.A.data_ptr(), self.B.data_ptr(), self.r, float(self.alpha))


def qlora_linear_workspace_bytes(L: QLoraLinear, M: int) -> int:
    cl = L.c()
    return int(load_library().qlora_linear_workspace_bytes(ctypes.byref(cl), M))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def qlora_linear_fwd(L: QLoraLinear, X: torch.Tensor, Y=None, XA=None, ws=None):
    """qlora_linear_fwd: returns (Y bf16 [M, N], XA fp32 [M, r])."""
    lib = load_library()
    M = X.shape[0]
    dev = X.device
    _need(X, torch.bfloat16, (M, L.W0.K), "X")
    Y = torch.empty(M, L.W0.N, dtype=torch.bfloat16, device=dev) if Y is None else Y
    XA = torch.empty(M, L.r, dtype=torch.float32, device=dev) if XA is None else XA
    ws = _workspace(qlora_linear_workspace_bytes(L, M), dev) if ws is None else ws
    cl = L.c()
    st = lib.qlora_linear_fwd(ctypes.byref(cl), X.data_ptr(), M, Y.data_ptr(), XA.data_ptr(), ws.data_ptr(),
                              ws.numel(), _stream(dev))
    _check("qlora_linear_fwd", st)
    return Y, XA


def qlora_linear_fwd_static(L: QLoraLinear, X: torch.Tensor, Y=None, XA=None):
    """qlora_linear_fwd_static: as qlora_linear_fwd with the library's static
    per-GPU scratch instead of a workspace; returns (Y, XA)."""
    lib = load_library()
    M = X.shape[0]
    dev = X.device
    _need(X, torch.bfloat16, (M, L.W0.K), "X")
    Y = torch.empty(M, L.W0.N, dtype=torch.bfloat16, device=dev) if Y is None else Y
    XA = torch.empty(M, L.r, dtype=torch.float32, device=dev) if XA is None else XA
    cl = L.c()
    _check("qlora_linear_fwd_static", lib.qlora_linear_fwd_static(ctypes.byref(cl), X.data_ptr(), M, Y.data_ptr(),
                                                                  XA.data_ptr(), _stream(dev)))
    return Y, XA


def debug_force_arch(name: Optional[str]):
    """qlora_debug_force_arch: pretend every device is `name` (None: the real one)."""
    _check("qlora_debug_force_arch",
           load_library().qlora_debug_force_arch(None if name is None else name.encode()))


def qlora_linear_bwd(L: QLoraLinear, dY: torch.Tensor, X: torch.Tensor, XA: torch.Tensor, dX=None, dA=None,
                     dB=None, ws=None):
    """qlora_linear_bwd: returns (dX bf16 [M, K], dA bf16 [r, K], dB bf16 [N, r])."""
    lib = load_library()
    M = X.shape[0]
    dev = X.device
    _need(dY, torch.bfloat16, (M, L.W0.N), "dY")
    dX = torch.empty(M, L.W0.K, dtype=torch.bfloat16, device=dev) if dX is None else dX
    dA = torch.empty_like(L.A) if dA is None else dA
    dB = torch.empty_like(L.B) if dB is None else dB
    ws = _workspace(qlora_linear_workspace_bytes(L, M), dev) if ws is None else ws
    cl = L.c()
    st = lib.qlora_linear_bwd(ctypes.byref(cl), dY.data_ptr(), X.data_ptr(), XA.data_ptr(), M, dX.data_ptr(),
                              dA.data_ptr(), dB.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev))
    _check("qlora_linear_bwd", st)
    return dX, dA, dB


@dataclass
class QLoraGrouped:
    """Several adapters over one input, packed: W0 the NF4 weight of the stacked
    rows [W_0; W_1; ...], A the stacked A_g [r_total, K], Bs one B_g [N_g, r_g]
    per group, alphas one alpha per group."""
    W0: Nf4Weight
    A: torch.Tensor
    Bs: list
    alphas: list

    @property
    def rs(self):
        return [int(B.shape[1]) for B in self.Bs]

    @property
    def Ns(self):
        return [int(B.shape[0]) for B in self.Bs]

    def c(self) -> CGrouped:
        q = CGrouped()
        q.W0 = self.W0.c()
        q.A = self.A.data_ptr()
        q.G = len(self.Bs)
        for g, B in enumerate(self.Bs):
            q.B[g] = B.data_ptr()
            q.N[g] = int(B.shape[0])
            q.r[g] = int(B.shape[1])
            q.alpha[g] = float(self.alphas[g])
        return q


def qlora_grouped_workspace_bytes(Q: QLoraGrouped, M: int) -> int:
    cq = Q.c()
    return int(load_library().qlora_grouped_workspace_bytes(ctypes.byref(cq), M))


def qlora_grouped_fwd(Q: QLoraGrouped, X: torch.Tensor, Y=None, XA=None, ws=None):
    """qlora_grouped_fwd: returns (Y bf16 [M, N_total], XA fp32 [M, r_total])."""
    lib = load_library()
    M, dev = X.shape[0], X.device
    Y = torch.empty(M, Q.W0.N, dtype=torch.bfloat16, device=dev) if Y is None else Y
    XA = torch.empty(M, sum(Q.rs), dtype=torch.float32, device=dev) if XA is None else XA
    ws = _workspace(qlora_grouped_workspace_bytes(Q, M), dev) if ws is None else ws
    cq = Q.c()
    _check("qlora_grouped_fwd", lib.qlora_grouped_fwd(ctypes.byref(cq), X.data_ptr(), M, Y.data_ptr(),
                                                      XA.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev)))
    return Y, XA


def qlora_grouped_bwd(Q: QLoraGrouped, dY: torch.Tensor, X: torch.Tensor, XA: torch.Tensor, ws=None):
    """qlora_grouped_bwd: returns (dX bf16 [M, K], dA bf16 [r_total, K], [dB_g bf16 [N_g, r_g]])."""
    lib = load_library()
    M, dev = X.shape[0], X.device
    dX = torch.empty(M, Q.W0.K, dtype=torch.bfloat16, device=dev)
    dA = torch.empty_like(Q.A)
    dBs = [torch.empty_like(B) for B in Q.Bs]
    ptrs = (ctypes.c_void_p * 8)(*[b.data_ptr() for b in dBs])
    ws = _workspace(qlora_grouped_workspace_bytes(Q, M), dev) if ws is None else ws
    cq = Q.c()
    _check("qlora_grouped_bwd", lib.qlora_grouped_bwd(ctypes.byref(cq), dY.data_ptr(), X.data_ptr(), XA.data_ptr(),
                                                      M, dX.data_ptr(), dA.data_ptr(), ptrs, ws.data_ptr(),
                                                      ws.numel(), _stream(dev)))
    return dX, dA, dBs


def rmsnorm_fwd(X: torch.Tensor, w: torch.Tensor, eps: float, Y: Optional[torch.Tensor] = None,
                rstd: Optional[torch.Tensor] = None):
    """rmsnorm_fwd: returns (Y bf16 [M, D], rstd fp32 [M])."""
    lib = load_library()
    M, D = X.shape
    Y = torch.empty_like(X) if Y is None else Y
    rstd = torch.empty(M, dtype=torch.float32, device=X.device) if rstd is None else rstd
    _check("rmsnorm_fwd", lib.rmsnorm_fwd(_ptr(X), _ptr(w), M, D, float(eps), _ptr(Y), _ptr(rstd),
                                          _stream(X.device)))
    return Y, rstd


def rmsnorm_bwd(dY: torch.Tensor, X: torch.Tensor, w: torch.Tensor, rstd: torch.Tensor, want_dw: bool = True,
                dX: Optional[torch.Tensor] = None, dw: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None):
    """rmsnorm_bwd: returns (dX bf16 [M, D], dw fp32 [D] or None)."""
    lib = load_library()
    M, D = X.shape
    dX = torch.empty_like(X) if dX is None else dX
    if want_dw and dw is None:
        dw = torch.empty(D, dtype=torch.float32, device=X.device)
    nbytes = lib.rmsnorm_bwd_workspace_bytes(M, D) if want_dw else 0
    if ws is None:
        ws = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=X.device)
    _check("rmsnorm_bwd", lib.rmsnorm_bwd(_ptr(dY), _ptr(X), _ptr(w), _ptr(rstd), M, D, _ptr(dX),
                                          _ptr(dw) if want_dw else None, _ptr(ws), ws.numel(),
                                          _stream(X.device)))
    return dX, (dw if want_dw else None)


IGNORE_INDEX = -100


def qlora_linear_ce_workspace_bytes(T: int, D: int, V: int, chunk: int, want_dx: bool = True) -> int:
    return int(load_library().qlora_linear_ce_workspace_bytes(T, D, V, chunk, 1 if want_dx else 0))


def qlora_linear_ce(X: torch.Tensor, W: torch.Tensor, targets: torch.Tensor, ignore_index: int = IGNORE_INDEX,
                    chunk: int = 1024, want_dx: bool = True, want_token_loss: bool = False,
                    dX: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """qlora_linear_ce: returns (loss fp32 [1], token_loss fp32 [T] or None, dX bf16 [T, D] or None)."""
    lib = load_library()
    T, D = X.shape
    V = W.shape[0]
    loss = torch.empty(1, dtype=torch.float32, device=X.device)
    tl = torch.empty(T, dtype=torch.float32, device=X.device) if want_token_loss else None
    if want_dx and dX is None:
        dX = torch.empty_like(X)
    if ws is None:
        nbytes = lib.qlora_linear_ce_workspace_bytes(T, D, V, chunk, 1 if want_dx else 0)
        ws = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=X.device)
    _check("qlora_linear_ce", lib.qlora_linear_ce(_ptr(X), T, D, _ptr(W), V, _ptr(targets), int(ignore_index),
                                                  int(chunk), _ptr(loss), _ptr(tl) if tl is not None else None,
                                                  _ptr(dX) if want_dx else None, _ptr(ws), ws.numel(),
                                                  _stream(X.device)))
    return loss, tl, (dX if want_dx else None)


def qlora_merge(L: QLoraLinear, dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None):
    """qlora_merge: the layer as one 16-bit weight [N, K], round16(deq(W0) + s B A)."""
    lib = load_library()
    if out is None:
        out = torch.empty(L.W0.N, L.W0.K, dtype=dtype, device=L.A.device)
    code = QLORA_DTYPE_F16 if out.dtype == torch.float16 else QLORA_DTYPE_BF16
    cl = L.c()
    _check("qlora_merge", lib.qlora_merge(ctypes.byref(cl), code, out.data_ptr(), _stream(out.device)))
    return out


# ------------------------------------------------------------------ MLP

@dataclass
class QLoraMlp:
    gate: QLoraLinear
    up: QLoraLinear
    down: QLoraLinear

    def c(self) -> CMlp:
        return CMlp(self.gate.c(), self.up.c(), self.down.c())

    @property
    def D(self) -> int:
        return self.gate.W0.K

    @property
    def I(self) -> int:  # noqa: E743
        return self.gate.W0.N


@dataclass
class MlpSaved:
    G: torch.Tensor
    U: torch.Tensor
    XA_g: torch.Tensor
    XA_u: torch.Tensor
    HA_d: torch.Tensor

    def c(self) -> CMlpSaved:
        return CMlpSaved(self.G.data_ptr(), self.U.data_ptr(), self.XA_g.data_ptr(), self.XA_u.data_ptr(),
                         self.HA_d.data_ptr())


def qlora_mlp_workspace_bytes(P: QLoraMlp, M: int) -> int:
    cm = P.c()
    return int(load_library().qlora_mlp_workspace_bytes(ctypes.byref(cm), M))


def alloc_mlp_saved(P: QLoraMlp, M: int, device) -> MlpSaved:
    f32, bf = torch.float32, torch.bfloat16
    return MlpSaved(torch.empty(M, P.I, dtype=bf, device=device), torch.empty(M, P.I, dtype=bf, device=device),
                    torch.empty(M, P.gate.r, dtype=f32, device=device),
                    torch.empty(M, P.up.r, dtype=f32, device=device),
                    torch.empty(M, P.down.r, dtype=f32, device=device))


def qlora_mlp_fwd(P: QLoraMlp, X: torch.Tensor, Y=None, saved: Optional[MlpSaved] = None, ws=None):
    """qlora_mlp_fwd: returns (Y bf16 [M, D], MlpSaved)."""
    lib = load_library()
    M = X.shape[0]
    dev = X.device
    _need(X, torch.bfloat16, (M, P.D), "X")
    Y = torch.empty(M, P.D, dtype=torch.bfloat16, device=dev) if Y is None else Y
    saved = alloc_mlp_saved(P, M, dev) if saved is None else saved
    ws = _workspace(qlora_mlp_workspace_bytes(P, M), dev) if ws is None else ws
    cm, cs = P.c(), saved.c()
    st = lib.qlora_mlp_fwd(ctypes.byref(cm), X.data_ptr(), M, Y.data_ptr(), ctypes.byref(cs), ws.data_ptr(),
                           ws.numel(), _stream(dev))
    _check("qlora_mlp_fwd", st)
    return Y, saved


def qlora_mlp_rmsnorm_workspace_bytes(P: QLoraMlp, M: int) -> int:
    cm = P.c()
    return int(load_library().qlora_mlp_rmsnorm_workspace_bytes(ctypes.byref(cm), M))


def qlora_mlp_fwd_rmsnorm(P: QLoraMlp, X: torch.Tensor, norm_w: torch.Tensor, eps: float, Y=None,
                          saved: Optional[MlpSaved] = None, rstd=None, want_xn: bool = False, Xn=None, ws=None):
    """qlora_mlp_fwd_rmsnorm: returns (Y, MlpSaved, rstd fp32 [M], Xn bf16 [M, D] or None)."""
    lib = load_library()
    M = X.shape[0]
    dev = X.device
    _need(X, torch.bfloat16, (M, P.D), "X")
    _need(norm_w, torch.bfloat16, (P.D,), "norm_w")
    Y = torch.empty(M, P.D, dtype=torch.bfloat16, device=dev) if Y is None else Y
    saved = alloc_mlp_saved(P, M, dev) if saved is None else saved
    rstd = torch.empty(M, dtype=torch.float32, device=dev) if rstd is None else rstd
    if want_xn and Xn is None:
        Xn = torch.empty(M, P.D, dtype=torch.bfloat16, device=dev)
    ws = _workspace(qlora_mlp_rmsnorm_workspace_bytes(P, M), dev) if ws is None else ws
    cm, cs = P.c(), saved.c()
    st = lib.qlora_mlp_fwd_rmsnorm(ctypes.byref(cm), X.data_ptr(), norm_w.data_ptr(), float(eps), M, Y.data_ptr(),
                                   ctypes.byref(cs), rstd.data_ptr(), None if Xn is None else Xn.data_ptr(),
                                   ws.data_ptr(), ws.numel(), _stream(dev))
    _check("qlora_mlp_fwd_rmsnorm", st)
    return Y, saved, rstd, Xn


def qlora_mlp_bwd(P: QLoraMlp, dY: torch.Tensor, X: torch.Tensor, saved: MlpSaved, dX=None, grads=None, ws=None):
    """qlora_mlp_bwd: returns (dX bf16 [M, D], dict of the six LoRA gradients)."""
    lib = load_library()
    M = X.shape[0]
    dev = X.device
    _need(dY, torch.bfloat16, (M, P.D), "dY")
    dX = torch.empty(M, P.D, dtype=torch.bfloat16, device=dev) if dX is None else dX
    if grads is None:
        grads = dict(dA_g=torch.empty_like(P.gate.A), dB_g=torch.empty_like(P.gate.B),
                     dA_u=torch.empty_like(P.up.A), dB_u=torch.empty_like(P.up.B),
                     dA_d=torch.empty_like(P.down.A), dB_d=torch.empty_like(P.down.B))
    ws = _workspace(qlora_mlp_workspace_bytes(P, M), dev) if ws is None else ws
    cm, cs = P.c(), saved.c()
    cg = CMlpGrads(*[grads[k].data_ptr() for k in ("dA_g", "dB_g", "dA_u", "dB_u", "dA_d", "dB_d")])
    st = lib.qlora_mlp_bwd(ctypes.byref(cm), dY.data_ptr(), X.data_ptr(), ctypes.byref(cs), M, dX.data_ptr(),
                           ctypes.byref(cg), ws.data_ptr(), ws.numel(), _stream(dev))
    _check("qlora_mlp_bwd", st)
    return dX, grads


# ------------------------------------------------------------------ tracing

GEMM_KINDS = {0: "fwd", 1: "fwd_swiglu", 2: "bwd_dx", 3: "bwd_dh_swiglu", 4: "bwd_dx_dual"}
# trace kind = GEMM kind + 8 when the bf16-staged kernel (bgemm_kernel) ran
GEMM_KERNELS = {k: "qgemm_kernel" for k in GEMM_KINDS}
GEMM_KERNELS.update({k + 8: "bgemm_kernel" for k in GEMM_KINDS})
GEMM_KERNELS.update({k + 16: "skinny_kernel" for k in GEMM_KINDS})


class LaunchTrace:
    """qlora_trace_install: HIP-event timing of every GEMM launch on its stream.

    Events are created with hipEventCreate from the HIP runtime that torch
    already loaded; ``durations()`` returns (kind, milliseconds) per launch.
    """

    def __init__(self, capacity: int = 4096):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.cap = capacity
        self.begin = (ctypes.c_void_p * capacity)()
        self.end = (ctypes.c_void_p * capacity)()
        for arr in (self.begin, self.end):
            for i in range(capacity):
                h = ctypes.c_void_p()
                if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                arr[i] = h
        self.kinds = (ctypes.c_int32 * capacity)()
        self.count = ctypes.c_int32(0)

    def __enter__(self):
        self.count.value = 0
        _check("qlora_trace_install", load_library().qlora_trace_install(
            self.begin, self.end, self.kinds, self.cap, ctypes.byref(self.count)))
        return self

    def __exit__(self, *exc):
        load_library().qlora_trace_install(None, None, None, 0, None)
        return False

    def durations(self):
        out = []
        for i in range(min(self.count.value, self.cap)):
            ms = ctypes.c_float()
            if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.begin[i], self.end[i]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append((GEMM_KINDS.get(self.kinds[i] & 7, str(self.kinds[i])), float(ms.value)))
        return out

    def launches(self):
        """(kind, kernel name, milliseconds) per traced GEMM launch."""
        return [(kind, GEMM_KERNELS.get(self.kinds[i], "?"), ms)
                for i, (kind, ms) in enumerate(self.durations())]

    def close(self):
        for arr in (self.begin, self.end):
            for h in arr:
                self.hip.hipEventDestroy(h)
