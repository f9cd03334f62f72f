"""NF4 blockwise-absmax quantization, double quantization and dequantization.

TEST INFRASTRUCTURE ONLY (see the package docstring): the plain CPU oracle.

The pages only name the format: QLoRA stores the frozen base weights as 4-bit
NormalFloat, a quarter of the 16-bit footprint ("LLM Fine-Tuning in 2026:
Unsloth vs QLoRA vs Liger-Kernel", FAQ on LoRA vs QLoRA; "Speed Up Fine-Tuning
2x with Unsloth", item 1).  The block size (64), the fp32 or double-quantized
absmax and the codebook given as an input table fix the rest.  Readings taken
where the pages are silent:

* blocks are 64 consecutive elements of one weight row (K % 64 == 0);
* the normalised value is the correctly rounded fp32 quotient w / absmax;
* the code is the nearest codebook entry, ties going to the lower index,
  i.e. the number of codebook midpoints (computed exactly in fp64) that the
  normalised value strictly exceeds;
* an all-zero block gets the index of the codebook's 0.0 entry everywhere;
* byte p of the packed codes holds element 2p in bits 0-3 and element 2p+1 in
  bits 4-7 (row-major element order);
* double quantization: the flat absmax vector is cut into groups of
  ``dq_group`` (256) consecutive entries, the last group may be shorter; each
  group stores S = fp32(max / 255) and 8-bit codes round_half_even(fp32(a / S))
  clamped to 255 (0 when S == 0); the 4-bit codes are computed from the exact
  absmax, and dequantization uses fp32(code8 * S);
* a dequantized element is fp32(codebook[q] * absmax'); its bf16 export rounds
  that to nearest even.
"""
from __future__ import annotations

import numpy as np

_ROWS_PER_CHUNK = 4096


def zero_index(codebook: np.ndarray) -> int:
    cb = np.asarray(codebook, np.float32)
    z = np.flatnonzero(cb == 0.0)
    if z.size != 1:
        raise ValueError("codebook must contain exactly one 0.0 entry")
    return int(z[0])


def midpoints(codebook: np.ndarray) -> np.ndarray:
    """(c_j + c_{j+1}) / 2 in fp64; exact because both are fp32 of modest range."""
    cb = np.asarray(codebook, np.float32).astype(np.float64)
    return (cb[:-1] + cb[1:]) / 2.0


def absmax_blocks(W: np.ndarray, blocksize: int = 64) -> np.ndarray:
    """Per-block max |w| (fp32, exact in any order), flat over row-major blocks."""
    W = np.asarray(W, np.float32)
    N, K = W.shape
    if K % blocksize:
        raise ValueError("K must be a multiple of the block size")
    return np.abs(W.reshape(N * K // blocksize, blocksize)).max(axis=1)


def codes_of_block_values(w: np.ndarray, a: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """4-bit indices of the values ``w`` [nb, bs] in blocks with absmax ``a`` [nb]."""
    w = np.asarray(w, np.float32)
    a = np.asarray(a, np.float32)
    mids = midpoints(codebook)
    q = np.full(w.shape, zero_index(codebook), np.uint8)
    nz = a != 0
    if np.any(nz):
        # correctly rounded fp32 quotient (IEEE division in float32)
        n = w[nz] / a[nz][:, None]
        # number of midpoints strictly below n, compared exactly in fp64
        q[nz] = np.searchsorted(mids, n.astype(np.float64), side="left").astype(np.uint8)
    return q


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """Element 2p -> low nibble of byte p, element 2p+1 -> high nibble."""
    flat = np.asarray(q, np.uint8).reshape(-1)
    return (flat[0::2] | (flat[1::2] << np.uint8(4))).astype(np.uint8)


def unpack_nibbles(codes: np.ndarray, n: int) -> np.ndarray:
    codes = np.asarray(codes, np.uint8).reshape(-1)
    q = np.empty(2 * codes.size, np.uint8)
    q[0::2] = codes & np.uint8(0x0F)
    q[1::2] = codes >> np.uint8(4)
    return q[:n]


def double_quantize(absmax: np.ndarray, group: int = 256):
    """8-bit linear codes of the absmax vector with one fp32 scale per group."""
    a = np.asarray(absmax, np.float32).reshape(-1)
    ngroups = -(-a.size // group)
    scales = np.empty(ngroups, np.float32)
    codes8 = np.empty(a.size, np.uint8)
    for g in range(ngroups):
        seg = a[g * group:(g + 1) * group]
        S = np.float32(seg.max()) / np.float32(255.0)
        scales[g] = S
        if S == 0:
            codes8[g * group:(g + 1) * group] = 0
        else:
            ratio = seg / S  # fp32 quotient
            codes8[g * group:(g + 1) * group] = np.minimum(np.rint(ratio), 255.0).astype(np.uint8)
    return codes8, scales


def dq_absmax(codes8: np.ndarray, scales: np.ndarray, group: int = 256) -> np.ndarray:
    """a' = fp32(code8 * S) for every block."""
    c = np.asarray(codes8, np.uint8).reshape(-1)
    S = np.repeat(np.asarray(scales, np.float32), group)[: c.size]
    return (c.astype(np.float32) * S).astype(np.float32)


def quantize(W: np.ndarray, codebook: np.ndarray, blocksize: int = 64, dq_group: int = 0):
    """Quantize an fp32 [N, K] weight.

    Returns a dict with ``codes`` (uint8 [N*K/2]) and either ``absmax`` (fp32
    [N*K/blocksize]) when ``dq_group == 0``, or ``absmax_q`` (uint8) and
    ``absmax_scale`` (fp32 [ceil(nblocks / dq_group)]) otherwise.
    """
    W = np.asarray(W, np.float32)
    N, K = W.shape
    if K % blocksize:
        raise ValueError("K must be a multiple of the block size")
    absmax = absmax_blocks(W, blocksize)
    bpr = K // blocksize
    codes = np.empty(N * K // 2, np.uint8)
    for r0 in range(0, N, _ROWS_PER_CHUNK):
        r1 = min(N, r0 + _ROWS_PER_CHUNK)
        blocks = W[r0:r1].reshape(-1, blocksize)
        q = codes_of_block_values(blocks, absmax[r0 * bpr:r1 * bpr], codebook)
        codes[r0 * K // 2:r1 * K // 2] = pack_nibbles(q)
    out = dict(codes=codes, N=N, K=K, blocksize=blocksize, dq_group=dq_group)
    if dq_group:
        out["absmax_q"], out["absmax_scale"] = double_quantize(absmax, dq_group)
    else:
        out["absmax"] = absmax
    return out


def effective_absmax(qw: dict) -> np.ndarray:
    if qw["dq_group"]:
        return dq_absmax(qw["absmax_q"], qw["absmax_scale"], qw["dq_group"])
    return np.asarray(qw["absmax"], np.float32)


def dequantize(qw: dict, codebook: np.ndarray, rows: slice | None = None) -> np.ndarray:
    """fp32 [N, K] (or the selected rows): fp32(codebook[q] * absmax')."""
    N, K, bs = qw["N"], qw["K"], qw["blocksize"]
    rows = rows or slice(0, N)
    r0, r1 = rows.start or 0, N if rows.stop is None else rows.stop
    cb = np.asarray(codebook, np.float32)
    a = effective_absmax(qw)[r0 * K // bs:r1 * K // bs]
    q = unpack_nibbles(qw["codes"][r0 * K // 2:r1 * K // 2], (r1 - r0) * K)
    vals = cb[q].reshape(-1, bs) * a[:, None]  # fp32 * fp32 -> fp32
    return vals.astype(np.float32).reshape(r1 - r0, K)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def dequantize_bf16(qw: dict, codebook: np.ndarray, rows: slice | None = None) -> np.ndarray:
    return to_bf16_bits(dequantize(qw, codebook, rows))
