"""Helpers for the GPU parity tests: host <-> device moves and error metrics.

Inputs come from ``synth`` (seeded, shared by both sides); expected values come
only from ``oracle``.  The HIP side is reached only through the C ABI binding.
"""
import numpy as np
import torch

import synth
from oracle import nf4 as onf4
from oracle import qlora as oq

REL_TOL = 1e-2  # relative Frobenius error bound for every floating-point output


def bf16_dev(u16: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).to(device)


def f32_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def u16_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def f64_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return oq.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.double().numpy()


def rel_fro(gpu: torch.Tensor, ref: np.ndarray) -> float:
    g = f64_host(gpu)
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(g - ref)
    if den == 0:
        return 0.0 if num == 0 else float("inf")
    return float(num / den)


def assert_close(name, gpu, ref, tol=REL_TOL):
    e = rel_fro(gpu, ref)
    print("  %-6s rel_fro=%.3e" % (name, e), flush=True)
    assert e <= tol, "%s: relative Frobenius error %.3e > %.1e" % (name, e, tol)
    return e


def quantize_both(W: np.ndarray, cb: np.ndarray, dq: int, q):
    """GPU quantization through the ABI, and the oracle's, of the same weight."""
    Wd = f32_dev(W)
    qw = q.nf4_quantize(Wd, f32_dev(cb), dq_group=dq)
    ow = onf4.quantize(W, cb, dq_group=dq)
    return qw, ow


def assert_codes_equal(qw, ow):
    assert np.array_equal(qw.codes.cpu().numpy(), ow["codes"])
    if ow["dq_group"]:
        assert np.array_equal(qw.absmax_q.cpu().numpy(), ow["absmax_q"])
        assert np.array_equal(qw.absmax_scale.cpu().numpy().view(np.uint32), ow["absmax_scale"].view(np.uint32))
    else:
        assert np.array_equal(qw.absmax.cpu().numpy().view(np.uint32), ow["absmax"].view(np.uint32))


def make_linear(q, W, A_u16, B_u16, alpha, cb, dq):
    """Quantize W on both sides; returns (QLoraLinear, oracle dequantized fp64 W)."""
    qw, ow = quantize_both(W, cb, dq, q)
    assert_codes_equal(qw, ow)
    L = q.QLoraLinear(qw, bf16_dev(A_u16), bf16_dev(B_u16), alpha)
    return L, onf4.dequantize(ow, cb).astype(np.float64)


class Guarded:
    """Output tensors for the parity tests, each carved out of its own buffer
    between two guard bands of a fixed byte pattern; the output itself starts
    with the same pattern.  ``check()`` (after the calls) asserts that no
    kernel wrote outside its output: every guard byte must be unchanged."""

    PAD = 4096   # bytes before and after each output (keeps 256-byte alignment)
    FILL = 0xA5

    def __init__(self, device="cuda"):
        self.device = device
        self.bufs = []

    def empty(self, shape, dtype):
        shape = tuple(int(d) for d in shape)
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        body = (n + 255) // 256 * 256
        buf = torch.full((self.PAD + body + self.PAD,), self.FILL, dtype=torch.uint8, device=self.device)
        self.bufs.append((buf, n))
        return buf[self.PAD:self.PAD + n].view(dtype).view(shape)

    def empty_like(self, t):
        return self.empty(t.shape, t.dtype)

    def check(self):
        torch.cuda.synchronize()
        for i, (buf, n) in enumerate(self.bufs):
            head, tail = buf[:self.PAD], buf[self.PAD + n:]
            assert bool((head == self.FILL).all()), "output %d: bytes written before its start" % i
            assert bool((tail == self.FILL).all()), "output %d: bytes written past its end" % i

